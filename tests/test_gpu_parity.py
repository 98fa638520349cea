"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Each step is checked on inputs both sides receive from the seeded generator:
  * gating on given float32 logits -> indices bit-exact, weights to 2e-6;
  * the fused router on integer-valued inputs (exact in float32 in any
    summation order) -> logits and indices bit-exact, ties included;
  * permutation of given top-k indices -> counts, offsets, rows, drops bit-exact;
  * expert FFNs on given rows and combine on given expert outputs -> within
    the output tolerance (1e-5 float32, 1e-2 bf16, relative to max |oracle|);
  * the whole layer on Gaussian inputs -> within tolerance, with routing
    flips (tokens whose oracle and GPU logits rank experts differently)
    counted and required to be near ties.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_gating_amd as moe
import workloads
from gpu_harness import DEV, TOL, rel_err, run_forward, to_dev, token_choice_flips

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().to("cpu").float().numpy() if t.dtype != torch.int32 else t.detach().cpu().numpy()


# ---------------------------------------------------------------------------
# gating on given logits
# ---------------------------------------------------------------------------

GATE_CASES = [("topk_softmax", 8, 2), ("topk_softmax", 256, 8), ("topk_softmax", 64, 6), ("softmax_topk", 16, 4),
              ("switch", 16, 1), ("topk_softmax", 5, 5), ("topk_softmax", 200, 64), ("topk_softmax", 256, 256)]


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("gating,E,k", GATE_CASES)
def test_gate_from_logits_bit_exact(gating, E, k, ties):
    T = 777
    lg = workloads.random_logits(T, E, seed=100 + E + k, ties=ties)
    spec = workloads.LayerSpec("gate", 90, T=T, d=64, E=E, k=k, F=64, gating=gating, act="swiglu", dtype="bf16",
                               capacity_factor=1.25 if gating == "switch" else 0.0)
    cfg = moe.config_from_spec(spec)
    r = moe.alloc_routing(cfg, DEV)
    moe.moe_route_from_logits(cfg, lg.to(DEV), moe.make_routing(r))
    torch.cuda.synchronize()
    idx, w = oracle.route_topk(lg.numpy(), k, gating)
    assert np.array_equal(_np(r["topk_idx"]).reshape(T, k), idx)
    np.testing.assert_allclose(_np(r["topk_w"]).reshape(T, k), w, rtol=2e-6, atol=1e-30)


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("T,E", [(1000, 16), (8192, 64), (300, 7), (16384, 4), (20000, 8)])  # > 16384: column not cached in LDS
def test_expert_choice_select_bit_exact(T, E, ties):
    lg = workloads.random_logits(T, E, seed=200 + E, ties=ties)
    spec = workloads.LayerSpec("ec", 91, T=T, d=64, E=E, k=0, F=64, gating="expert_choice", act="swiglu",
                               dtype="bf16", capacity_factor=1.0)
    cfg = moe.config_from_spec(spec)
    C = moe.moe_capacity(cfg)
    assert C == oracle.capacity(1.0, T, E)
    r = moe.alloc_routing(cfg, DEV)
    moe.moe_route_from_logits(cfg, lg.to(DEV), moe.make_routing(r))
    torch.cuda.synchronize()
    ec_idx, ec_score = oracle.route_expert_choice(lg.numpy(), C)
    assert np.array_equal(_np(r["topk_idx"]).reshape(E, C), ec_idx)
    np.testing.assert_allclose(_np(r["topk_w"]).reshape(E, C), ec_score, rtol=1e-5, atol=1e-30)


# ---------------------------------------------------------------------------
# fused router on exact (integer-valued) inputs
# ---------------------------------------------------------------------------

INT_SPECS = [s.replace(name=s.name + "_int", inputs="integer") for s in workloads.SMALL] + [
    # the LDS-staged router tiles with 128 and 256 expert columns, 32- and 64-token blocks
    workloads.DEEPSEEK_SHARED_BF16.replace(name="router_e256_int", T=333, d=512, E=256, k=8, F=64, F_shared=0,
                                           inputs="integer"),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="router_e128_int", T=300, d=1024, E=128, k=6, F=64, F_shared=0,
                                           inputs="integer"),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="router_e256_t32768_int", T=32768, d=128, E=256, k=8, F=64,
                                           F_shared=0, inputs="integer"),
    # one router block that also permutes its selections inside moe_forward
    # (bf16 token choice, T <= 16, E <= 16): the Mixtral decode router at
    # d = 4096 (16 waves), and a Switch batch whose capacity drops tokens
    workloads.MIXTRAL_DECODE_BF16.replace(name="one_block_decode_d4096_int", F=256, inputs="integer"),
    workloads.SWITCH_TOP1_BF16.replace(name="one_block_switch_drops_int", T=16, d=512, E=4, F=256,
                                       capacity_factor=1.0, capacity_group=0, inputs="integer"),
]


# The router variants the full-size layers run, at their real K depth and
# token counts (integer inputs keep every product and sum exact): the
# 16-wave K split (d >= 4096, Mixtral prefill router), the 8-wave one
# (1024 <= d < 4096), the LDS-staged tile router with 256 expert columns at
# d = 7168 over 8192 tokens (DeepSeek-style router), and with 64 columns at
# the expert-choice layer's shape.
ROUTER_DEPTH_SPECS = [
    workloads.MIXTRAL_PREFILL_BF16.replace(name="router_16_waves_d4096_t4096_int", inputs="integer"),
    workloads.SWITCH_TOP1_BF16.replace(name="router_8_waves_d2048_e16_int", d=2048, inputs="integer"),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="router_tile_d7168_e256_t8192_int", inputs="integer"),
    workloads.EXPERT_CHOICE_BF16.replace(name="router_tile_d2048_e64_t8192_ec_int", inputs="integer"),
]


# Routers of at most 8 experts with d % 64 == 0 pair two 32-wide K segments
# in one MFMA (the diagonal blocks of the product); waves with no K step
# (d = 64, 192), uneven K splits (d = 1088, 4160), fewer than 8 experts and
# ragged token tails.
PAIR_SPECS = [
    workloads.MIXTRAL_PREFILL_BF16.replace(name="pair_e8_d64_t37_int", T=37, d=64, F=64, inputs="integer"),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="pair_e3_d192_t1000_int", T=1000, d=192, E=3, F=64, inputs="integer"),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="pair_e1_d128_t50_int", T=50, d=128, E=1, k=1, F=64,
                                           inputs="integer"),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="pair_e5_k3_d1088_t333_softmax_topk_int", T=333, d=1088, E=5, k=3,
                                           F=64, gating="softmax_topk", inputs="integer"),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="pair_e8_d4160_t100_int", T=100, d=4160, F=64, inputs="integer"),
    workloads.SWITCH_TOP1_BF16.replace(name="pair_switch_e8_d512_int", T=2048, d=512, E=8, F=64, inputs="integer"),
]


# float32 routers: up to 64 experts, lanes split each expert's dot product
# over S = 64 / (E rounded up to a power of two) chunk sets (E = 1: S = 64;
# E = 3: S = 16; E = 64: S = 1); more experts, one lane per expert.
F32_ROUTER_SPECS = [
    workloads.BASIC_TOP2_F32.replace(name="router_f32_e1_int", T=70, d=64, E=1, k=1, inputs="integer"),
    workloads.BASIC_TOP2_F32.replace(name="router_f32_e3_d272_int", T=130, d=272, E=3, k=2, inputs="integer"),
    workloads.BASIC_TOP2_F32.replace(name="router_f32_e64_int", T=99, d=128, E=64, k=4, inputs="integer"),
    workloads.BASIC_TOP2_F32.replace(name="router_f32_e80_int", T=50, d=96, E=80, k=3, inputs="integer"),
]


@pytest.mark.parametrize("spec", INT_SPECS + ROUTER_DEPTH_SPECS + PAIR_SPECS + F32_ROUTER_SPECS, ids=lambda s: s.name)
def test_fused_route_bit_exact_on_exact_inputs(spec):
    inp = workloads.make_inputs(spec, experts=False)
    dinp = to_dev(inp)
    cfg = moe.config_from_spec(spec)
    r = moe.alloc_routing(cfg, DEV)
    moe.moe_route(cfg, dinp["x"], moe.make_weights(dinp), moe.make_routing(r))
    torch.cuda.synchronize()
    lg = oracle.logits(inp["x"], inp["wg"], inp["bg"])
    assert np.array_equal(_np(r["logits"]), lg)
    if spec.gating == "expert_choice":
        C = moe.moe_capacity(cfg)
        ec_idx, ec_score = oracle.route_expert_choice(lg, C)
        assert np.array_equal(_np(r["topk_idx"]).reshape(spec.E, C), ec_idx)
        np.testing.assert_allclose(_np(r["topk_w"]).reshape(spec.E, C), ec_score, rtol=1e-5, atol=1e-30)
    else:
        idx, w = oracle.route_topk(lg, spec.k, spec.gating)
        assert np.array_equal(_np(r["topk_idx"]).reshape(spec.T, spec.k), idx)
        np.testing.assert_allclose(_np(r["topk_w"]).reshape(spec.T, spec.k), w, rtol=2e-6, atol=1e-30)


# ---------------------------------------------------------------------------
# permutation on given indices
# ---------------------------------------------------------------------------

PERM_CASES = [  # T, E, k, capacity_factor, group
    (777, 8, 2, 0.0, 0), (4096, 16, 1, 1.25, 1024), (8192, 256, 8, 0.0, 0), (640, 16, 1, 1.25, 320),
    (1000, 16, 1, 1.25, 0), (130, 64, 6, 0.0, 0), (64, 1, 1, 0.0, 0), (1, 4, 4, 0.0, 0),
    # at and past the limits of the one-workgroup path (T*k <= 16384; chunk tables of nc = ceil(T / 64)
    # rows of E + 1 entries, 16 bytes each, <= 40 KiB)
    (16384, 8, 1, 0.0, 0), (1280, 127, 2, 0.0, 0), (1280, 128, 2, 0.0, 0), (1344, 128, 2, 0.0, 0),
    (20000, 16, 1, 1.25, 1024), (3000, 64, 6, 0.0, 0),
    # the most experts the permutation accepts (1024): one-workgroup path, three-kernel path, capacity drops
    (100, 1024, 4, 0.0, 0), (3000, 1024, 2, 0.0, 0), (4096, 1024, 1, 1.25, 1024)]


def _small_path(T, E, k):
    nc = (T + 63) // 64
    return T * k <= 16384 and nc * (E + 1) * 16 <= 40 * 1024


@pytest.mark.parametrize("T,E,k,cf,group", PERM_CASES)
def test_permute_bit_exact(T, E, k, cf, group):
    gating = "switch" if cf > 0 else "topk_softmax"
    idx = workloads.random_topk_idx(T, E, k, seed=300 + T + E, skew=1.1 if E > 1 else 0.0)
    spec = workloads.LayerSpec("perm", 92, T=T, d=128, E=E, k=k, F=64, gating=gating, act="swiglu", dtype="bf16",
                               capacity_factor=cf, capacity_group=group)
    cfg = moe.config_from_spec(spec)
    x = workloads.make_inputs(spec, experts=False)["x"]
    r = moe.alloc_routing(cfg, DEV)
    r["topk_idx"].copy_(idx.reshape(-1).to(DEV))
    x_perm = torch.full((T * k, spec.d), -7.0, dtype=torch.bfloat16, device=DEV)
    ws = moe.alloc_workspace(cfg, moe.STAGE_PERMUTE, DEV)
    moe.moe_timing_reset()
    moe.moe_timing_enable(True)
    moe.moe_permute(cfg, x.to(DEV), moe.make_routing(r), x_perm, ws)
    torch.cuda.synchronize()
    names = moe.moe_kernel_names()
    launched = {n for i, n in enumerate(names) if moe.moe_timing_read(i)[1]}
    moe.moe_timing_enable(False)
    assert ("permute_small" in launched) == _small_path(T, E, k)
    assert ("permute_count" in launched) != _small_path(T, E, k)
    cap = oracle.capacity(cf, group if group else T, E) if cf > 0 else 0
    ref = oracle.permute(idx.numpy(), E, cap, group)
    n = ref["kept"]
    assert np.array_equal(_np(r["counts"]), ref["counts"])
    assert np.array_equal(_np(r["offsets"]), ref["offsets"])
    assert np.array_equal(_np(r["row_token"])[:n], ref["row_token"])
    assert np.array_equal(_np(r["slot_row"]).reshape(T, k), ref["slot_row"])
    assert torch.equal(x_perm[:n].cpu(), x[torch.from_numpy(ref["row_token"]).long()])
    assert (x_perm[n:] == -7.0).all()  # rows past the kept ones are untouched


def test_expert_choice_permute_bit_exact():
    T, E = 1000, 16
    lg = workloads.random_logits(T, E, seed=7)
    spec = workloads.EXPERT_CHOICE_BF16.replace(name="ecp", T=T, d=256, E=E, F=192)
    cfg = moe.config_from_spec(spec)
    C = moe.moe_capacity(cfg)
    ec_idx, _ = oracle.route_expert_choice(lg.numpy(), C)
    x = workloads.make_inputs(spec, experts=False)["x"]
    r = moe.alloc_routing(cfg, DEV)
    r["topk_idx"].copy_(torch.from_numpy(ec_idx.reshape(-1)).to(DEV))
    x_perm = torch.empty((E * C, spec.d), dtype=torch.bfloat16, device=DEV)
    ws = moe.alloc_workspace(cfg, moe.STAGE_PERMUTE, DEV)
    moe.moe_permute(cfg, x.to(DEV), moe.make_routing(r), x_perm, ws)
    torch.cuda.synchronize()
    assert np.array_equal(_np(r["counts"]), np.full(E, C))
    assert np.array_equal(_np(r["offsets"]), np.arange(E + 1) * C)
    assert np.array_equal(_np(r["row_token"]), ec_idx.reshape(-1))
    sr = np.full((T, E), -1)
    for e in range(E):
        sr[ec_idx[e], e] = e * C + np.arange(C)
    assert np.array_equal(_np(r["slot_row"]).reshape(T, E), sr)
    assert torch.equal(x_perm.cpu(), x[torch.from_numpy(ec_idx.reshape(-1)).long()])


# ---------------------------------------------------------------------------
# expert FFNs and combine on given inputs
# ---------------------------------------------------------------------------

FFN_SPECS = workloads.SMALL + [workloads.MIXTRAL_DECODE_BF16.replace(name="mixtral_decode_d512", d=512, F=1024)]
# Long K loops on few tiles.  The 256-row tiles with at least 64 K steps
# split the partial last round of tiles along K (2 or 4 parts, float32
# partials added by the last part); the other shapes run unsplit.
LONG_K_SPECS = [
    workloads.MIXTRAL_PREFILL_BF16.replace(name="long_k_prefill_tiles", T=1000, d=2048, F=1024),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="long_k_small_m_tiles", T=1200, d=4096, E=16, k=1, F=512),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="long_k_decode_tiles", T=16, d=2048, F=2048),
    # decode gate/up on K tiles of 128 needs d % 128 == 0; d = 448 takes the 64 path
    workloads.MIXTRAL_PREFILL_BF16.replace(name="decode_tiles_k_not_multiple_of_128", T=16, d=448, F=1024),
]
SPLITK_SPECS = [
    workloads.MIXTRAL_PREFILL_BF16.replace(name="splitk_gemm1", T=700, d=4096, F=256),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="splitk_gemm2_4_parts", T=700, d=256, F=8192),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="splitk_shared_expert", T=520, d=4096, E=64, F=64, F_shared=256),
    # 128-row tiles, about 100 down-projection tiles for 256 slots and a K loop of 160 tiles: 5 parts a tile,
    # more split work items than slots
    workloads.MIXTRAL_PREFILL_BF16.replace(name="splitk_parts_exceed_slots", T=1250, d=1024, E=25, k=1, F=10240),
]
# Combinations the ABI accepts beyond the six layers: expert biases on the
# bf16 MFMA path (ReLU and GELU epilogues, 256-, 128- and 32-row tiles), the
# float32 SwiGLU and GELU experts, softmax-then-top-k gating without
# renormalisation end to end, and float32 shared-expert and expert-choice
# layers.
ABI_SPECS = [
    workloads.BASIC_TOP2_F32.replace(name="relu_bias_bf16_256_row_tiles", dtype="bf16", T=2000, d=256, F=384),
    workloads.BASIC_TOP2_F32.replace(name="relu_bias_bf16_128_row_tiles", dtype="bf16", T=1200, d=256, E=16, k=2,
                                     F=8192),
    workloads.BASIC_TOP2_F32.replace(name="relu_bias_bf16_decode", dtype="bf16", T=16, d=256, F=384),
    workloads.SWITCH_TOP1_BF16.replace(name="gelu_bias_bf16_switch", T=640, d=256, F=640, capacity_group=320,
                                       expert_bias=True),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="gelu_bf16_top2_no_bias", act="gelu", T=900, d=256, F=320),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="swiglu_f32", dtype="f32", T=300, d=128, F=192),
    workloads.SWITCH_TOP1_BF16.replace(name="gelu_f32_switch", dtype="f32", T=640, d=128, F=256,
                                       capacity_group=320),
    workloads.SWITCH_TOP1_BF16.replace(name="gelu_bias_f32_top2", dtype="f32", gating="topk_softmax", k=2,
                                       T=300, d=128, F=256, capacity_factor=0.0, capacity_group=0,
                                       expert_bias=True),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="softmax_topk_bf16", gating="softmax_topk", T=500, d=256, E=16,
                                           k=4, F=256),
    workloads.BASIC_TOP2_F32.replace(name="softmax_topk_f32_relu_bias", gating="softmax_topk", T=203),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="shared_expert_f32", dtype="f32", T=200, d=128, E=32, k=4, F=64,
                                           F_shared=96),
    workloads.EXPERT_CHOICE_BF16.replace(name="expert_choice_f32", dtype="f32", T=500, d=128, E=8, F=96),
    # several shared experts, summed ([yj-zh] DeepSeekMoELayer): the down
    # projection reads their [S][d][Fs] blocks as slices of its K axis
    workloads.DEEPSEEK_SHARED_BF16.replace(name="two_shared_experts", T=520, d=384, E=64, F=256, F_shared=320,
                                           num_shared=2),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="three_shared_experts_decode", T=16, d=512, E=16, k=4, F=128,
                                           F_shared=192, num_shared=3),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="two_shared_experts_f32", dtype="f32", T=200, d=128, E=32, k=4,
                                           F=64, F_shared=96, num_shared=2),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="two_shared_experts_split_k", T=520, d=512, E=64, F=64,
                                           F_shared=2048, num_shared=2),
]
# Tile paths of the 256-row SwiGLU gate/up GEMM: K % 128 == 0 takes the
# direct-to-LDS kernel, other K the register-staged one; an expert (and a
# shared expert) of more than 8 m-tiles runs its tiles in bands of 8 m-tiles.
# Zipf-skewed routing gives the direct-to-LDS kernel tiles of a few rows
# next to full ones, also in a last round of tiles split along K.
TILE_SPECS = [
    workloads.MIXTRAL_PREFILL_BF16.replace(name="prefill_tiles_k_not_multiple_of_128", T=1000, d=320, F=384),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="banded_tiles_shared_expert", T=3000, d=256, E=16, k=2, F=64,
                                           F_shared=512),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="light_tiles_skewed", T=1024, d=512, E=32, k=8, F=256, F_shared=0),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="light_tiles_split_k", T=1024, d=4096, E=16, k=4, F=128,
                                           F_shared=0),
    # T*k > 16384: the three-kernel permutation, whose scan also builds the
    # tile plan in the forward pass (Zipf-skewed, interleaved light tiles)
    workloads.DEEPSEEK_SHARED_BF16.replace(name="three_kernel_permutation_plan_in_scan", T=2200, d=256, E=64, k=8,
                                           F=128, F_shared=256),
]
FFN_SPECS = FFN_SPECS + LONG_K_SPECS + SPLITK_SPECS + ABI_SPECS + TILE_SPECS


@pytest.mark.parametrize("spec", FFN_SPECS, ids=lambda s: s.name)
def test_expert_ffn_matches_oracle(spec):
    inp = workloads.make_inputs(spec)
    dinp = to_dev(inp)
    cfg = moe.config_from_spec(spec)
    lg = oracle.logits(inp["x"], inp["wg"], inp["bg"])
    if spec.gating == "expert_choice":
        C = moe.moe_capacity(cfg)
        ec_idx, _ = oracle.route_expert_choice(lg, C)
        counts = np.full(spec.E, C, np.int32)
        row_token = ec_idx.reshape(-1)
    else:
        idx, _ = oracle.route_topk(lg, spec.k, spec.gating)
        cap = oracle.capacity(spec.capacity_factor, spec.capacity_group, spec.E) if spec.gating == "switch" else 0
        p = oracle.permute(idx, spec.E, cap, spec.capacity_group)
        counts, row_token = p["counts"], p["row_token"]
    _check_ffn(spec, inp, dinp, counts, row_token)


def _check_ffn(spec, inp, dinp, counts, row_token):
    """moe_expert_ffn on rows x[row_token] grouped by `counts` against the oracle's expert FFNs."""
    cfg = moe.config_from_spec(spec)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    r = moe.alloc_routing(cfg, DEV)
    r["counts"].copy_(torch.from_numpy(counts).to(DEV))
    r["offsets"].copy_(torch.from_numpy(offsets).to(DEV))
    a_max = r["row_token"].numel()
    x_perm = torch.zeros((a_max, spec.d), dtype=spec.torch_dtype, device=DEV)
    x_perm[:len(row_token)] = dinp["x"][torch.from_numpy(row_token).long().to(DEV)]
    y_perm = torch.full((a_max, spec.d), 3.0, dtype=spec.torch_dtype, device=DEV)
    y_shared = torch.empty((spec.T, spec.d), dtype=spec.torch_dtype, device=DEV) if spec.F_shared else None
    ws = moe.alloc_workspace(cfg, moe.STAGE_FFN, DEV)
    moe.moe_expert_ffn(cfg, x_perm, dinp["x"], moe.make_routing(r), moe.make_weights(dinp), y_perm, y_shared, ws)
    torch.cuda.synchronize()
    n = int(offsets[-1])
    got = _np(y_perm)
    for e in range(spec.E):
        rows = slice(offsets[e], offsets[e + 1])
        if offsets[e] == offsets[e + 1]:
            continue
        ref = oracle.expert_ffn(spec.act, inp["x"][torch.from_numpy(row_token[rows]).long()], inp["w1"][e],
                                None if inp["w3"] is None else inp["w3"][e], inp["w2"][e],
                                None if inp["b1"] is None else inp["b1"][e],
                                None if inp["b2"] is None else inp["b2"][e])
        assert rel_err(got[rows], ref) <= TOL[spec.dtype], f"expert {e}"
    assert (got[n:] == 3.0).all()  # rows past the routed ones are untouched
    if spec.F_shared:
        ref = oracle.shared_ffn(inp["x"], inp["ws1"], inp["ws3"], inp["ws2"])
        assert rel_err(_np(y_shared), ref) <= TOL[spec.dtype]


# Row counts just past and below multiples of the tile height: each expert's
# rows are cut into equal m-tiles of whole MFMA row blocks, and a wave skips
# the blocks past its tile's last row.  256-row tiles (ragged plan with a
# one-row expert among the others' m-tiles; plain plan) and 128-row tiles.
BALANCED_CASES = [
    (workloads.MIXTRAL_PREFILL_BF16.replace(name="balanced_256_ragged_plan", T=1024, d=512, E=4, F=512),
     [257, 1030, 1, 760]),
    (workloads.MIXTRAL_PREFILL_BF16.replace(name="balanced_256", T=2048, d=512, E=4, F=512),
     [513, 1030, 17, 2536]),
    (workloads.MIXTRAL_PREFILL_BF16.replace(name="balanced_128", T=2048, d=2048, E=16, k=1, F=512),
     [129, 1, 257, 0, 300, 64, 96, 200, 33, 31, 150, 128, 159, 161, 99, 240]),
]


@pytest.mark.parametrize("spec,counts", BALANCED_CASES, ids=lambda c: getattr(c, "name", ""))
def test_expert_ffn_balanced_tiles(spec, counts):
    assert sum(counts) == spec.T * spec.k
    inp = workloads.make_inputs(spec)
    rng = np.random.default_rng(7)
    row_token = rng.integers(0, spec.T, spec.T * spec.k).astype(np.int32)
    _check_ffn(spec, inp, to_dev(inp), np.asarray(counts, np.int32), row_token)


@pytest.mark.parametrize("spec", [SPLITK_SPECS[0], SPLITK_SPECS[2], SPLITK_SPECS[3]], ids=lambda s: s.name)
def test_split_k_forward_is_deterministic_and_matches_oracle(spec):
    inp = workloads.make_inputs(spec)
    dinp = to_dev(inp)
    y1, routing = run_forward(spec, dinp)
    y2, _ = run_forward(spec, dinp)
    assert torch.equal(y1, y2)  # partials are added in part order, whatever the arrival order
    _check_layer(spec, inp, y1, routing, oracle.forward(spec, inp))


# Few tokens: each token's columns are split over several waves (ranges of
# whole 8-element chunks; d = 1088 leaves a range of 544 and one of 544).
COMBINE_SPECS = workloads.SMALL + [
    workloads.MIXTRAL_DECODE_BF16.replace(name="combine_split_columns", T=5, d=1088),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="combine_split_columns_shared", T=3, d=4096, E=16, k=4),
    workloads.BASIC_TOP2_F32.replace(name="combine_split_columns_f32", T=2, d=1536),
    workloads.EXPERT_CHOICE_BF16.replace(name="combine_split_columns_ec", T=64, d=2048, E=4),
    # expert choice over many tokens: two column ranges per token, ranges of
    # 68 chunks (a wave's second pass takes 4 of them)
    workloads.EXPERT_CHOICE_BF16.replace(name="combine_ec_two_ranges", T=3000, d=1088, E=16),
]


@pytest.mark.parametrize("spec", COMBINE_SPECS, ids=lambda s: s.name)
def test_combine_matches_oracle(spec):
    inp = workloads.make_inputs(spec, experts=False)
    cfg = moe.config_from_spec(spec)
    lg = workloads.random_logits(spec.T, spec.E, seed=17)
    r = moe.alloc_routing(cfg, DEV)
    g = torch.Generator().manual_seed(5)
    a_max = r["row_token"].numel()
    y_perm = torch.randn((a_max, spec.d), generator=g).to(spec.torch_dtype)
    y_shared = torch.randn((spec.T, spec.d), generator=g).to(spec.torch_dtype) if spec.F_shared else None
    if spec.gating == "expert_choice":
        C = moe.moe_capacity(cfg)
        ec_idx, ec_score = oracle.route_expert_choice(lg.numpy(), C)
        r["topk_w"].copy_(torch.from_numpy(ec_score.reshape(-1)).to(DEV))
        sr = np.full((spec.T, spec.E), -1, np.int32)
        for e in range(spec.E):
            sr[ec_idx[e], e] = e * C + np.arange(C)
        r["slot_row"].copy_(torch.from_numpy(sr.reshape(-1)).to(DEV))
        ref = oracle.combine_expert_choice(ec_idx, ec_score, y_perm.float().numpy(), spec.T,
                                           None if y_shared is None else y_shared.float().numpy())
    else:
        idx, w = oracle.route_topk(lg.numpy(), spec.k, spec.gating)
        cap = oracle.capacity(spec.capacity_factor, spec.capacity_group, spec.E) if spec.gating == "switch" else 0
        p = oracle.permute(idx, spec.E, cap, spec.capacity_group)
        r["topk_w"].copy_(torch.from_numpy(w.reshape(-1)).to(DEV))
        r["slot_row"].copy_(torch.from_numpy(p["slot_row"].reshape(-1)).to(DEV))
        ref = oracle.combine_topk(w, p["slot_row"], y_perm.float().numpy()[:max(p["kept"], 1)],
                                  None if y_shared is None else y_shared.float().numpy())
    y = torch.empty((spec.T, spec.d), dtype=spec.torch_dtype, device=DEV)
    moe.moe_combine(cfg, y_perm.to(DEV), None if y_shared is None else y_shared.to(DEV), moe.make_routing(r), y)
    torch.cuda.synchronize()
    tol = 1e-6 if spec.dtype == "f32" else 4e-3  # only the final rounding to the output dtype differs
    assert rel_err(_np(y), ref) <= tol


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def _check_layer(spec, inp, y, routing, ref):
    """Compare a GPU forward with the oracle's, excluding near-tie routing flips."""
    T = spec.T
    gpu_lg = _np(routing["logits"])
    or_lg = ref["logits"]
    ok = np.ones(T, bool)
    if spec.gating == "expert_choice":
        C = ref["capacity"]
        g_idx = _np(routing["topk_idx"]).reshape(spec.E, C)
        o_idx = ref["ec_idx"]
        dl = float(np.abs(gpu_lg.astype(np.float64) - or_lg).max())
        for e in range(spec.E):
            gs, os_ = set(g_idx[e].tolist()), set(o_idx[e].tolist())
            if gs != os_:
                col = np.sort(or_lg[:, e].astype(np.float64))[::-1]
                assert col[C - 1] - col[C] <= 4 * dl + 1e-30, f"expert {e} selection differs beyond a near tie"
                for t in gs ^ os_:
                    ok[t] = False
    else:
        k = spec.k
        flips, near, dl = token_choice_flips(_np(routing["topk_idx"]), ref["topk_idx"], gpu_lg, or_lg, k)
        assert near.all(), f"routing flips that are not near ties: {flips[~near]}"
        ok[flips] = False
        if ref["capacity"] > 0 and len(flips):
            # a flip shifts the positions of later tokens of the same (group, expert)
            G = spec.capacity_group or T
            gi = _np(routing["topk_idx"]).reshape(T, k)
            oi = ref["topk_idx"]
            touched = {(t // G, e) for t in flips for e in list(gi[t]) + list(oi[t])}
            for t in range(T):
                if any((t // G, e) in touched for e in list(gi[t]) + list(oi[t])):
                    ok[t] = False
        if not len(flips):
            assert np.array_equal(_np(routing["counts"]), ref["counts"])
            assert np.array_equal(_np(routing["slot_row"]).reshape(T, k), ref["slot_row"])
    assert ok.mean() > 0.95
    err = rel_err(_np(y)[ok], ref["y64"][ok])
    assert err <= TOL[spec.dtype], f"max rel error {err}"
    return (~ok).sum()


@pytest.mark.parametrize("spec", workloads.SMALL + ABI_SPECS + TILE_SPECS, ids=lambda s: s.name)
def test_forward_matches_oracle(spec):
    inp = workloads.make_inputs(spec)
    y, routing = run_forward(spec, to_dev(inp))
    ref = oracle.forward(spec, inp)
    _check_layer(spec, inp, y, routing, ref)


@pytest.mark.parametrize("spec", INT_SPECS, ids=lambda s: s.name)
def test_forward_integer_inputs_routing_bit_exact(spec):
    inp = workloads.make_inputs(spec)
    y, routing = run_forward(spec, to_dev(inp))
    ref = oracle.forward(spec, inp)
    assert np.array_equal(_np(routing["logits"]), ref["logits"])
    if spec.gating == "expert_choice":
        assert np.array_equal(_np(routing["topk_idx"]).reshape(spec.E, -1), ref["ec_idx"])
    else:
        assert np.array_equal(_np(routing["topk_idx"]).reshape(spec.T, spec.k), ref["topk_idx"])
        assert np.array_equal(_np(routing["slot_row"]).reshape(spec.T, spec.k), ref["slot_row"])
    assert np.array_equal(_np(routing["counts"]), ref["counts"])
    assert np.array_equal(_np(routing["offsets"]), ref["offsets"])
    n = int(ref["offsets"][-1])
    assert np.array_equal(_np(routing["row_token"])[:n], ref["row_token"])
    assert rel_err(_np(y), ref["y64"]) <= TOL[spec.dtype]


def test_forward_is_deterministic():
    spec = workloads.SMALL[4]
    dinp = to_dev(workloads.make_inputs(spec))
    y1, r1 = run_forward(spec, dinp)
    y2, r2 = run_forward(spec, dinp)
    assert torch.equal(y1, y2)
    for key in r1:
        assert torch.equal(r1[key], r2[key]), key


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def test_all_ties_route_to_lowest_experts():
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="ties", T=100, d=128, F=128, k=3)
    inp = workloads.make_inputs(spec)
    inp["wg"] = torch.zeros_like(inp["wg"])
    y, routing = run_forward(spec, to_dev(inp))
    idx = _np(routing["topk_idx"]).reshape(spec.T, 3)
    assert (idx == np.array([0, 1, 2])).all()
    np.testing.assert_allclose(_np(routing["topk_w"]), 1.0 / 3.0, rtol=1e-6)
    ref = oracle.forward(spec, inp)
    assert rel_err(_np(y), ref["y64"]) <= TOL["bf16"]


def test_one_expert_takes_every_token_and_others_stay_empty():
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="skewed", T=700, d=128, F=256, E=8, k=1,
                                                  router_bias="normal")
    inp = workloads.make_inputs(spec)
    inp["bg"] = torch.tensor([0, 0, 0, 0, 0, 1e4, 0, 0], dtype=torch.float32)
    y, routing = run_forward(spec, to_dev(inp))
    assert _np(routing["counts"]).tolist() == [0, 0, 0, 0, 0, 700, 0, 0]
    ref = oracle.forward(spec, inp)
    assert rel_err(_np(y), ref["y64"]) <= TOL["bf16"]


@pytest.mark.parametrize("T", [0, 1, 63, 65])
def test_tiny_and_empty_batches(T):
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name=f"T{T}", T=T, d=128, F=128)
    inp = workloads.make_inputs(spec)
    y, routing = run_forward(spec, to_dev(inp))
    if T == 0:
        assert y.numel() == 0
        return
    ref = oracle.forward(spec, inp)
    _check_layer(spec, inp, y, routing, ref)


def test_k_equals_E_and_single_expert():
    for spec in (workloads.MIXTRAL_PREFILL_BF16.replace(name="kE", T=96, d=128, F=128, E=4, k=4),
                 workloads.BASIC_TOP2_F32.replace(name="E1", T=70, E=1, k=1)):
        inp = workloads.make_inputs(spec)
        y, routing = run_forward(spec, to_dev(inp))
        ref = oracle.forward(spec, inp)
        _check_layer(spec, inp, y, routing, ref)


def test_invalid_arguments_are_rejected_before_launch():
    spec = workloads.SMALL[2]
    cfg = moe.config_from_spec(spec)
    cfg.top_k = spec.E + 1
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_workspace_size(cfg)
    assert ei.value.status == 1
    cfg = moe.config_from_spec(spec)
    dinp = to_dev(workloads.make_inputs(spec))
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    y = torch.empty((spec.T, spec.d), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward(cfg, dinp["x"], moe.make_weights(dinp), y, None, ws)
    assert ei.value.status == 3


# The forward pass routes many experts (bf16 token choice, 128..256 experts,
# at least 1024 tokens) with a K-split router GEMM and a separate gating
# kernel.  Integer inputs keep the logits exact in any summation order, so
# they, the selections and the permutation must equal the oracle's bit for
# bit; sampled outputs within tolerance.
ROUTER_GEMM_SPECS = [
    workloads.DEEPSEEK_SHARED_BF16.replace(name="router_gemm_d7168_e256_int", T=2048, d=7168, F=64, F_shared=0,
                                           inputs="integer"),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="router_gemm_d4096_e128_int", T=1500, d=4096, E=128, k=6, F=64,
                                           F_shared=128, inputs="integer"),
]


@pytest.mark.parametrize("spec", ROUTER_GEMM_SPECS, ids=lambda s: s.name)
def test_forward_router_gemm_exact(spec):
    inp = workloads.make_inputs(spec)
    dinp = to_dev(inp)
    moe.moe_timing_reset()
    moe.moe_timing_enable(True)
    y, routing = run_forward(spec, dinp)
    names = moe.moe_kernel_names()
    launched = {n for i, n in enumerate(names) if moe.moe_timing_read(i)[1]}
    moe.moe_timing_enable(False)
    assert "route_gate" in launched
    lg = oracle.logits(inp["x"], inp["wg"], inp["bg"])
    assert np.array_equal(_np(routing["logits"]), lg)
    idx, w = oracle.route_topk(lg, spec.k, spec.gating)
    assert np.array_equal(_np(routing["topk_idx"]).reshape(spec.T, spec.k), idx)
    np.testing.assert_allclose(_np(routing["topk_w"]).reshape(spec.T, spec.k), w, rtol=2e-6, atol=1e-30)
    perm = oracle.permute(idx, spec.E)
    n = perm["kept"]
    assert np.array_equal(_np(routing["counts"]), perm["counts"])
    assert np.array_equal(_np(routing["row_token"])[:n], perm["row_token"])
    assert np.array_equal(_np(routing["slot_row"]).reshape(spec.T, spec.k), perm["slot_row"])
    toks = np.array([0, 1, spec.T // 3, spec.T // 2, spec.T - 2, spec.T - 1])
    ref = oracle.forward_tokens(spec, inp, toks, lg=lg)
    assert rel_err(_np(y)[toks], ref["y64"]) <= TOL[spec.dtype]
