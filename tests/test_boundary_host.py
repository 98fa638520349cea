"""Host-side checks of the C ABI library (no GPU needed): it loads, exports
every function include/moe.h declares, and rejects bad arguments on the host
before any launch."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_gating_amd as moe
from sparse_mixture_experts_gating_amd import binding
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = moe.load()
    names = _declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(binding.EXPORTS) == names


def test_kernel_names_listed():
    names = moe.moe_kernel_names()
    assert "gemm1_act" in names and "route" in names and "combine" in names


@pytest.mark.parametrize("spec", workloads.FULL + workloads.SMALL, ids=lambda s: s.name)
def test_capacity_and_workspace_for_every_workload(spec):
    cfg = moe.config_from_spec(spec)
    cap = moe.moe_capacity(cfg)
    if spec.gating == "switch":
        assert cap == int(spec.capacity_factor * spec.capacity_group / spec.E)
    elif spec.gating == "expert_choice":
        assert cap == int(spec.capacity_factor * spec.T / spec.E)
    else:
        assert cap == 0
    for stage in (moe.STAGE_FORWARD, moe.STAGE_PERMUTE, moe.STAGE_FFN):
        assert moe.moe_workspace_size(cfg, stage) >= 0
    assert moe.moe_workspace_size(cfg, moe.STAGE_FORWARD) >= moe.moe_workspace_size(cfg, moe.STAGE_FFN)


def _status(fn, *args):
    with pytest.raises(moe.MoEError) as ei:
        fn(*args)
    return ei.value.status


BAD = [
    (dict(top_k=0), 1), (dict(top_k=9), 1), (dict(num_experts=0), 1), (dict(d_model=0), 1),
    (dict(gating=7), 1), (dict(act=5), 1), (dict(dtype=3), 1), (dict(num_tokens=-1), 1),
    (dict(d_model=100), 2), (dict(d_ff=96), 2), (dict(num_experts=2000, top_k=1), 2),
]


@pytest.mark.parametrize("change,status", BAD)
def test_bad_configs_rejected(change, status):
    cfg = moe.config_from_spec(workloads.MIXTRAL_PREFILL_BF16)
    for k, v in change.items():
        setattr(cfg, k, v)
    assert _status(moe.moe_workspace_size, cfg, 0) == status
    assert "moe" not in moe.moe_last_error() or True


def test_switch_and_expert_choice_rules():
    cfg = moe.config_from_spec(workloads.SWITCH_TOP1_BF16)
    cfg.top_k = 2
    assert _status(moe.moe_capacity, cfg) == 1
    cfg = moe.config_from_spec(workloads.SWITCH_TOP1_BF16)
    cfg.capacity_group = 100  # not a multiple of 64
    assert _status(moe.moe_capacity, cfg) == 2
    cfg = moe.config_from_spec(workloads.SWITCH_TOP1_BF16)
    cfg.capacity_factor = 0.0
    assert _status(moe.moe_capacity, cfg) == 1
    cfg = moe.config_from_spec(workloads.EXPERT_CHOICE_BF16)
    cfg.capacity_factor = 0.001  # int(8192 * 0.001 / 64) = 0
    assert _status(moe.moe_capacity, cfg) == 1
    cfg = moe.config_from_spec(workloads.EXPERT_CHOICE_BF16)
    cfg.capacity_factor = 40.0  # C = 5120 > the select buffer
    assert _status(moe.moe_capacity, cfg) == 2


def test_null_pointers_rejected_without_a_gpu():
    spec = workloads.MIXTRAL_PREFILL_BF16
    cfg = moe.config_from_spec(spec)
    w = binding.moe_weights()
    r = binding.moe_routing()
    lib = moe.load()
    assert lib.moe_route(ctypes.byref(cfg), None, ctypes.byref(w), ctypes.byref(r), None) == 1
    assert b"x is NULL" in lib.moe_last_error()
    assert lib.moe_forward(ctypes.byref(cfg), ctypes.c_void_p(256), ctypes.byref(w), ctypes.c_void_p(256), None,
                           None, 0, None) == 1
    assert lib.moe_permute(ctypes.byref(cfg), None, None, None, None, 0, None) == 1
    assert lib.moe_combine(ctypes.byref(cfg), None, None, None, None, None) == 1
    # misaligned x
    assert lib.moe_route(ctypes.byref(cfg), ctypes.c_void_p(258), ctypes.byref(w), ctypes.byref(r), None) == 1
    assert b"aligned" in lib.moe_last_error()
    # router limited to 256 experts
    big = moe.config_from_spec(workloads.DEEPSEEK_SHARED_BF16)
    big.num_experts = 512
    assert lib.moe_route(ctypes.byref(big), ctypes.c_void_p(256), ctypes.byref(w), ctypes.byref(r), None) == 2


def test_empty_batch_is_a_no_op():
    cfg = moe.config_from_spec(workloads.MIXTRAL_PREFILL_BF16.replace(T=0))
    lib = moe.load()
    assert lib.moe_forward(ctypes.byref(cfg), None, None, None, None, None, 0, None) == 0


def test_permute_noalloc_rejects_before_any_device_call():
    """The allocation-free permutation refuses, on the host, a batch whose
    scratch exceeds its fixed array, and null routing buffers."""
    lib = moe.load()
    spec = workloads.DEEPSEEK_SHARED_BF16.replace(T=200000)
    cfg = moe.config_from_spec(spec)
    assert moe.moe_workspace_size(cfg, moe.STAGE_PERMUTE) > (8 << 20)
    r = binding.moe_routing(*([ctypes.c_void_p(256)] * 7))
    p = ctypes.c_void_p(256)
    assert lib.moe_permute_noalloc(ctypes.byref(cfg), p, ctypes.byref(r), p, None) == 2
    assert b"exceeds the fixed" in lib.moe_last_error()
    ok = moe.config_from_spec(workloads.DEEPSEEK_SHARED_BF16)
    assert moe.moe_workspace_size(ok, moe.STAGE_PERMUTE) <= (8 << 20)
    assert lib.moe_permute_noalloc(ctypes.byref(ok), p, None, p, None) == 1
    assert lib.moe_permute_noalloc(ctypes.byref(ok), None, ctypes.byref(r), p, None) == 1
