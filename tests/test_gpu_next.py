"""Parity of the rows built after the core path: router side outputs (aux
load-balancing loss, router z-loss), top-k capacity with a floor, and the
noisy top-k router, against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_gating_amd as moe
import workloads
from gpu_harness import DEV, TOL, rel_err, to_dev
from test_gpu_parity import _check_layer, _np

pytestmark = pytest.mark.gpu


def _losses_gpu(spec, lg, idx):
    cfg = moe.config_from_spec(spec)
    out = torch.empty(2 + spec.E, dtype=torch.float32, device=DEV)
    ws = moe.alloc_workspace(cfg, moe.STAGE_LOSSES, DEV)
    moe.moe_router_losses(cfg, lg.to(DEV), idx.to(DEV), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T,E,k", [(777, 8, 2), (8192, 256, 8), (4096, 16, 1), (100, 64, 6)])
def test_router_losses_match_oracle(T, E, k):
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="loss", T=T, d=64, E=E, k=k, F=64)
    lg = workloads.random_logits(T, E, seed=400 + E)
    idx, _ = oracle.route_topk(lg.numpy(), k, "topk_softmax")
    got = _losses_gpu(spec, lg, torch.from_numpy(idx))
    aux, z, P = oracle.router_losses(lg.numpy(), idx)
    assert abs(got[0] - aux) <= 1e-5 * abs(aux)
    assert abs(got[1] - z) <= 1e-5 * abs(z)
    np.testing.assert_allclose(got[2:], P, rtol=1e-5, atol=1e-7)


def test_router_losses_closed_form_uniform():
    T, E, k = 640, 16, 2
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="loss_u", T=T, d=64, E=E, k=k, F=64)
    lg = torch.zeros(T, E)
    idx = (torch.arange(T * k).reshape(T, k) % E).to(torch.int32)
    got = _losses_gpu(spec, lg, idx)
    assert abs(got[0] - 1.0) < 1e-6
    assert abs(got[1] - math.log(E) ** 2) < 1e-5


CAP_CASES = [  # T, E, k, cf, group, min_cap
    (1024, 16, 2, 1.0, 128, 0), (1000, 8, 2, 1.25, 0, 0), (768, 64, 6, 0.5, 256, 4), (512, 16, 4, 0.25, 64, 9)]


@pytest.mark.parametrize("T,E,k,cf,group,min_cap", CAP_CASES)
def test_topk_capacity_permute_bit_exact(T, E, k, cf, group, min_cap):
    idx = workloads.random_topk_idx(T, E, k, seed=500 + E + k, skew=1.2)
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="capk", T=T, d=128, E=E, k=k, F=64, capacity_factor=cf,
                                                  capacity_group=group, min_capacity=min_cap)
    cfg = moe.config_from_spec(spec)
    cap = moe.moe_capacity(cfg)
    assert cap == oracle.capacity_topk(cf, group or T, k, E, min_cap)
    x = workloads.make_inputs(spec, experts=False)["x"]
    r = moe.alloc_routing(cfg, DEV)
    r["topk_idx"].copy_(idx.reshape(-1).to(DEV))
    x_perm = torch.empty((T * k, spec.d), dtype=torch.bfloat16, device=DEV)
    ws = moe.alloc_workspace(cfg, moe.STAGE_PERMUTE, DEV)
    moe.moe_permute(cfg, x.to(DEV), moe.make_routing(r), x_perm, ws)
    torch.cuda.synchronize()
    ref = oracle.permute(idx.numpy(), E, cap, group)
    assert (ref["slot_row"] < 0).any()
    assert np.array_equal(_np(r["counts"]), ref["counts"])
    assert np.array_equal(_np(r["offsets"]), ref["offsets"])
    assert np.array_equal(_np(r["slot_row"]).reshape(T, k), ref["slot_row"])
    n = ref["kept"]
    assert np.array_equal(_np(r["row_token"])[:n], ref["row_token"])


def _run_steps(spec, dinp, noisy):
    """route (noisy or not) -> permute -> expert_ffn -> combine through the step entry points."""
    cfg = moe.config_from_spec(spec)
    r = moe.alloc_routing(cfg, DEV)
    rr = moe.make_routing(r)
    w = moe.make_weights(dinp)
    if noisy:
        moe.moe_route_noisy(cfg, dinp["x"], w, dinp["wn"], dinp["noise"], rr)
    else:
        moe.moe_route(cfg, dinp["x"], w, rr)
    a_max = r["row_token"].numel()
    x_perm = torch.empty((a_max, spec.d), dtype=spec.torch_dtype, device=DEV)
    moe.moe_permute(cfg, dinp["x"], rr, x_perm, moe.alloc_workspace(cfg, moe.STAGE_PERMUTE, DEV))
    y_perm = torch.empty_like(x_perm)
    y_sh = torch.empty((spec.T, spec.d), dtype=spec.torch_dtype, device=DEV) if spec.F_shared else None
    moe.moe_expert_ffn(cfg, x_perm, dinp["x"], rr, w, y_perm, y_sh, moe.alloc_workspace(cfg, moe.STAGE_FFN, DEV))
    y = torch.empty((spec.T, spec.d), dtype=spec.torch_dtype, device=DEV)
    moe.moe_combine(cfg, y_perm, y_sh, rr, y)
    torch.cuda.synchronize()
    return y, r


@pytest.mark.parametrize("spec", [
    workloads.MIXTRAL_PREFILL_BF16.replace(name="mixtral_small_cap", T=1000, d=256, F=384, capacity_factor=1.0,
                                           capacity_group=256),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="deepseek_small_cap", T=520, d=384, E=64, F=256, F_shared=320,
                                           capacity_factor=1.0, min_capacity=4),
], ids=lambda s: s.name)
def test_forward_with_topk_capacity(spec):
    inp = workloads.make_inputs(spec)
    y, routing = _run_steps(spec, to_dev(inp), noisy=False)
    ref = oracle.forward(spec, inp)
    assert (ref["slot_row"] < 0).any()  # capacity drops happen
    _check_layer(spec, inp, y, routing, ref)


@pytest.mark.parametrize("spec", [
    workloads.MIXTRAL_PREFILL_BF16.replace(name="noisy_int", T=500, d=256, E=64, k=6, F=64, noisy=True,
                                           inputs="integer", router_bias="normal"),
    workloads.BASIC_TOP2_F32.replace(name="noisy_f32_int", T=300, d=128, E=8, k=2, noisy=True, inputs="integer",
                                     router_bias="normal"),
], ids=lambda s: s.name)
def test_noisy_router_zero_noise_is_exact_on_integer_inputs(spec):
    inp = workloads.make_inputs(spec, experts=False)
    inp["noise"] = torch.zeros_like(inp["noise"])
    dinp = to_dev(inp)
    cfg = moe.config_from_spec(spec)
    r = moe.alloc_routing(cfg, DEV)
    moe.moe_route_noisy(cfg, dinp["x"], moe.make_weights(dinp), dinp["wn"], dinp["noise"], moe.make_routing(r))
    torch.cuda.synchronize()
    lg = oracle.logits_noisy(inp["x"], inp["wg"], inp["bg"], inp["wn"], inp["noise"])
    assert np.array_equal(_np(r["logits"]), lg)
    idx, w = oracle.route_topk(lg, spec.k, spec.gating)
    assert np.array_equal(_np(r["topk_idx"]).reshape(spec.T, spec.k), idx)
    np.testing.assert_allclose(_np(r["topk_w"]).reshape(spec.T, spec.k), w, rtol=2e-6)


@pytest.mark.parametrize("spec", [
    workloads.MIXTRAL_PREFILL_BF16.replace(name="noisy_mixtral_small", T=1000, d=256, F=384, noisy=True),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="noisy_deepseek_small", T=520, d=384, E=256, F=128, F_shared=128,
                                           noisy=True),
    workloads.BASIC_TOP2_F32.replace(name="noisy_basic_f32", noisy=True),
], ids=lambda s: s.name)
def test_noisy_forward_matches_oracle(spec):
    inp = workloads.make_inputs(spec)
    y, routing = _run_steps(spec, to_dev(inp), noisy=True)
    ref = oracle.forward(spec, inp)
    dl = np.abs(_np(routing["logits"]).astype(np.float64) - ref["logits"]).max()
    assert dl <= 1e-3 * np.abs(ref["logits"]).max()
    _check_layer(spec, inp, y, routing, ref)


# The forward pass loads the routed token rows inside the first GEMM; the
# step entry points gather them into x_perm first.  Same products in the
# same order: the outputs agree bit for bit (bf16 and float32 layers).
GATHER_SPECS = list(workloads.SMALL) + [
    workloads.BASIC_TOP2_F32.replace(name="fused_gather_f32_swiglu", T=300, d=128, F=192, act="swiglu",
                                     expert_bias=False),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="fused_gather_f32_shared", dtype="f32", T=200, d=128, E=16, k=3,
                                           F=96, F_shared=64),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="fused_gather_split_k", T=700, d=4096, F=256),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="fused_gather_small_m", T=300, d=2048, F=512),
    workloads.MIXTRAL_DECODE_BF16.replace(name="fused_gather_decode", d=512, F=1024),
    workloads.SWITCH_TOP1_BF16.replace(name="fused_gather_drops", T=1000, d=256, F=512),
]


@pytest.mark.parametrize("spec", GATHER_SPECS, ids=lambda s: s.name)
def test_forward_gather_in_gemm_equals_step_path(spec):
    from gpu_harness import run_forward
    dinp = to_dev(workloads.make_inputs(spec))
    y_fwd, r_fwd = run_forward(spec, dinp)
    y_steps, r_steps = _run_steps(spec, dinp, noisy=False)
    n = int(r_fwd["offsets"][-1])  # rows past the kept ones are unspecified
    assert torch.equal(r_fwd["offsets"], r_steps["offsets"])
    assert torch.equal(r_fwd["row_token"][:n], r_steps["row_token"][:n])
    assert torch.equal(y_fwd, y_steps)


# A batch that fits one router block (bf16 token choice, T <= 16, E <= 16):
# in moe_forward that block also permutes its selections and writes the tile
# plan, so no permutation or plan kernel runs.  Its routing buffers and output
# equal the step path's bit for bit (1024-, 512- and 256-thread router blocks;
# Switch drops; one token).
ONE_BLOCK_SPECS = [
    workloads.MIXTRAL_DECODE_BF16.replace(name="one_block_d4096", d=4096, F=256),
    workloads.MIXTRAL_DECODE_BF16.replace(name="one_block_d1024_k4", d=1024, E=16, k=4, F=256),
    workloads.MIXTRAL_DECODE_BF16.replace(name="one_block_d512_t7", T=7, d=512, F=256),
    workloads.MIXTRAL_DECODE_BF16.replace(name="one_block_t1", T=1, d=512, F=256),
    workloads.SWITCH_TOP1_BF16.replace(name="one_block_switch_drops", T=16, d=512, E=4, F=256, capacity_factor=1.0,
                                       capacity_group=0),
]


@pytest.mark.parametrize("spec", ONE_BLOCK_SPECS, ids=lambda s: s.name)
def test_one_block_router_permutes_its_own_selections(spec):
    from gpu_harness import run_forward
    dinp = to_dev(workloads.make_inputs(spec))
    moe.moe_timing_reset()
    moe.moe_timing_enable(True)
    y_fwd, r_fwd = run_forward(spec, dinp)
    names = moe.moe_kernel_names()
    launched = {n for i, n in enumerate(names) if moe.moe_timing_read(i)[1]}
    moe.moe_timing_enable(False)
    assert "route" in launched
    assert not launched & {"permute_small", "permute_count", "permute_scan", "permute_scatter", "tile_plan"}
    y_steps, r_steps = _run_steps(spec, dinp, noisy=False)
    n = int(r_fwd["offsets"][-1])
    for key in ("topk_idx", "topk_w", "counts", "offsets", "slot_row"):
        assert torch.equal(r_fwd[key], r_steps[key]), key
    assert torch.equal(r_fwd["row_token"][:n], r_steps["row_token"][:n])
    assert torch.equal(y_fwd, y_steps)
    if spec.gating == "switch":
        assert (r_fwd["slot_row"] < 0).any()  # the capacity dropped some tokens
