"""Seeded synthetic workloads for the sparse MoE layer forward pass.

This module holds layer shapes and the input recipe only (random draws,
bf16 rounding of inputs, the fixed router-logit skews).  It computes no step
of the layer, and it is the only code the oracle side and the HIP side share:
both receive the very same input bytes from it.

Recipe (the same for every workload):
  * one torch.Generator per tensor, seed = (100 * workload_id + tensor_id) * 4096 + expert;
  * x ~ N(0, 1); every weight ~ N(0, 1/fan_in) (std fan_in^-1/2);
  * expert and router biases ~ N(0, 0.01) (std 0.1), basic top-2 layer only;
  * Switch layer: a fixed per-expert router bias ~ N(0, 1.5) (std sqrt(1.5)),
    so that some experts overflow their capacity;
  * DeepSeek-style layer: router bias b_e = -1.1 * ln(rank_e) with rank a seeded
    permutation of 1..E, i.e. a Zipf(1.1) prior over experts;
  * float32 draws, then rounded to bf16 (round to nearest even) for bf16 layers.
  * noisy routers: noise projection ~ N(0, 1/d) and the standard-normal draw
    n [T, E] are inputs like any other (seeded);
  * "integer" inputs: x in {-2..2}, router weights in {-4..4}/8 and router
    bias in {-8..8}/8, so every router product and sum is exact in float32 in
    any order and routing, ties included, can be compared bit for bit.

The pages measure nothing on a public dataset; these seeded tensors stand in
for real activations and trained weights.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    wid: int            # workload id, part of every seed
    T: int              # tokens (batch * sequence)
    d: int              # d_model
    E: int              # routed experts
    k: int              # experts per token (token choice); 0 for expert choice
    F: int              # expert hidden width d_ff
    gating: str         # topk_softmax | softmax_topk | switch | expert_choice
    act: str            # relu | gelu | swiglu
    dtype: str          # f32 | bf16
    expert_bias: bool = False
    router_bias: str = "none"   # none | normal | skew | zipf
    F_shared: int = 0           # width of each always-on SwiGLU shared expert; 0 = none
    num_shared: int = 1         # shared experts (with F_shared > 0), summed
    capacity_factor: float = 0.0
    capacity_group: int = 0     # tokens per capacity group (sequence length); 0 = all tokens
    inputs: str = "gaussian"    # gaussian | integer
    min_capacity: int = 0       # lower bound of the token-choice capacity
    noisy: bool = False         # noisy top-k router: + softplus(x Wn^T) * n, n ~ N(0,1) given

    def replace(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


# The five layers of the benchmark suite, at full size.
BASIC_TOP2_F32 = LayerSpec("basic_top2_f32", 1, T=256, d=128, E=8, k=2, F=512,
                           gating="topk_softmax", act="relu", dtype="f32",
                           expert_bias=True, router_bias="normal")
SWITCH_TOP1_BF16 = LayerSpec("switch_top1_bf16", 2, T=4096, d=512, E=16, k=1, F=2048,
                             gating="switch", act="gelu", dtype="bf16", router_bias="skew",
                             capacity_factor=1.25, capacity_group=1024)
MIXTRAL_PREFILL_BF16 = LayerSpec("mixtral_8x7b_prefill_bf16", 3, T=4096, d=4096, E=8, k=2,
                                 F=14336, gating="topk_softmax", act="swiglu", dtype="bf16")
MIXTRAL_DECODE_BF16 = MIXTRAL_PREFILL_BF16.replace(name="mixtral_8x7b_decode_bf16", T=16)
DEEPSEEK_SHARED_BF16 = LayerSpec("deepseek_fine_grained_shared_bf16", 4, T=8192, d=7168, E=256,
                                 k=8, F=2048, gating="topk_softmax", act="swiglu", dtype="bf16",
                                 router_bias="zipf", F_shared=2048)
EXPERT_CHOICE_BF16 = LayerSpec("expert_choice_bf16", 5, T=8192, d=2048, E=64, k=0, F=1408,
                               gating="expert_choice", act="swiglu", dtype="bf16",
                               capacity_factor=1.0)

FULL = [BASIC_TOP2_F32, SWITCH_TOP1_BF16, MIXTRAL_PREFILL_BF16, MIXTRAL_DECODE_BF16,
        DEEPSEEK_SHARED_BF16, EXPERT_CHOICE_BF16]

# Reduced copies the oracle runs in seconds.  Each keeps the layer's structure
# (gating, activation, biases, shared expert, skew) and spans several GEMM
# tiles with a ragged tail (T, rows per expert and d_ff not tile multiples).
SMALL = [
    BASIC_TOP2_F32.replace(name="basic_top2_f32_ragged", T=203),
    SWITCH_TOP1_BF16.replace(name="switch_top1_bf16_small", T=2 * 320, d=256, F=640,
                             capacity_group=320),
    MIXTRAL_PREFILL_BF16.replace(name="mixtral_small_prefill", T=1000, d=256, F=384),
    MIXTRAL_PREFILL_BF16.replace(name="mixtral_small_decode", T=16, d=256, F=384),
    DEEPSEEK_SHARED_BF16.replace(name="deepseek_small", T=520, d=384, E=64, F=256, F_shared=320),
    EXPERT_CHOICE_BF16.replace(name="expert_choice_small", T=1000, d=256, E=16, F=192),
]

BY_NAME = {s.name: s for s in FULL + SMALL}


def _seed(spec: LayerSpec, tensor_id: int, expert: int = 0) -> int:
    return (100 * spec.wid + tensor_id) * 4096 + expert


def _randn(shape, seed, device, std=1.0):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t * std if std != 1.0 else t


def _randint(shape, lo, hi, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.int64).float()


def _per_expert(spec, tensor_id, shape, std, device):
    out = torch.empty((spec.E,) + tuple(shape), dtype=spec.torch_dtype, device=device)
    for e in range(spec.E):
        out[e] = _randn(shape, _seed(spec, tensor_id, e), device, std).to(spec.torch_dtype)
    return out


def make_inputs(spec: LayerSpec, device="cpu", experts: bool = True) -> dict:
    """Seeded inputs of one layer.

    Returns a dict of tensors on ``device``: x [T,d], wg [E,d], bg [E] float32 or
    None, w1 [E,F,d], w3 [E,F,d] (SwiGLU) or None, w2 [E,d,F], b1 [E,F] / b2
    [E,d] float32 or None, and ws1 [Fs,d], ws3 [Fs,d], ws2 [d,Fs] for one
    shared expert ([S,Fs,d], [S,Fs,d], [S,d,Fs] for S > 1 of them) or None.
    ``experts=False`` skips the expert weights.
    """
    dt = spec.torch_dtype
    T, d, E, F = spec.T, spec.d, spec.E, spec.F
    if spec.inputs == "integer":
        x = _randint((T, d), -2, 2, _seed(spec, 1), device).to(dt)
        wg = (_randint((E, d), -4, 4, _seed(spec, 2), device) / 8).to(dt)
    else:
        x = _randn((T, d), _seed(spec, 1), device).to(dt)
        wg = _randn((E, d), _seed(spec, 2), device, 1.0 / math.sqrt(d)).to(dt)
    bg = None
    if spec.router_bias == "normal":
        bg = _randn((E,), _seed(spec, 3), device, 0.1)
    elif spec.router_bias == "skew":
        bg = _randn((E,), _seed(spec, 3), device, math.sqrt(1.5))
    elif spec.router_bias == "zipf":
        g = torch.Generator(device="cpu")
        g.manual_seed(_seed(spec, 3))
        rank = torch.randperm(E, generator=g).double() + 1.0
        bg = (-1.1 * torch.log(rank)).float().to(device)
    if bg is not None and spec.inputs == "integer":
        bg = _randint((E,), -8, 8, _seed(spec, 3), device) / 8
    out = dict(x=x, wg=wg, bg=bg, w1=None, w3=None, w2=None, b1=None, b2=None,
               ws1=None, ws3=None, ws2=None, wn=None, noise=None)
    if spec.noisy:
        out["wn"] = _randn((E, d), _seed(spec, 4), device, 1.0 / math.sqrt(d)).to(dt)
        out["noise"] = _randn((T, E), _seed(spec, 5), device)
    if not experts:
        return out
    out["w1"] = _per_expert(spec, 10, (F, d), 1.0 / math.sqrt(d), device)
    if spec.act == "swiglu":
        out["w3"] = _per_expert(spec, 11, (F, d), 1.0 / math.sqrt(d), device)
    out["w2"] = _per_expert(spec, 12, (d, F), 1.0 / math.sqrt(F), device)
    if spec.expert_bias:
        out["b1"] = _randn((E, F), _seed(spec, 13), device, 0.1)
        out["b2"] = _randn((E, d), _seed(spec, 14), device, 0.1)
    if spec.F_shared:
        Fs, S = spec.F_shared, spec.num_shared
        # shared expert s is seeded like routed expert s; one expert keeps 2-D tensors
        def stack(tensor_id, shape, std):
            parts = [_randn(shape, _seed(spec, tensor_id, s), device, std).to(dt) for s in range(S)]
            return parts[0] if S == 1 else torch.stack(parts)
        out["ws1"] = stack(20, (Fs, d), 1.0 / math.sqrt(d))
        out["ws3"] = stack(21, (Fs, d), 1.0 / math.sqrt(d))
        out["ws2"] = stack(22, (d, Fs), 1.0 / math.sqrt(Fs))
    return out


def random_logits(T: int, E: int, seed: int, ties: bool = False, device="cpu"):
    """Float32 logits handed to both sides as an input (gating parity on equal logits).
    ``ties=True`` draws from a coarse grid, so equal logits (and -0.0/+0.0) occur."""
    if ties:
        g = _randint((T, E), -3, 3, seed, device) * 0.5
        neg_zero = _randint((T, E), 0, 1, seed + 1, device) > 0
        return torch.where((g == 0) & neg_zero, torch.full_like(g, -0.0), g)
    return _randn((T, E), seed, device, 2.0)


def random_topk_idx(T: int, E: int, k: int, seed: int, skew: float = 0.0, device="cpu"):
    """k distinct experts per token, drawn with a skewed prior (int32 [T, k]) -- an
    input for the permutation step given to both sides."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    prior = torch.exp(-skew * torch.log(torch.arange(1, E + 1, dtype=torch.float64)))
    idx = torch.multinomial(prior.expand(T, E), k, replacement=False, generator=g)
    return idx.to(torch.int32).to(device)
