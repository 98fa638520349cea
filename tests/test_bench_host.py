"""Host logic of bench.py: the algorithmic work per kernel and the bound it
implies (no GPU)."""
import bench
import workloads


def _counts(spec, rows):
    return [rows // spec.E] * spec.E


def test_expert_gemm_flops_add_up_to_active_flops():
    for spec in (workloads.MIXTRAL_PREFILL_BF16, workloads.DEEPSEEK_SHARED_BF16, workloads.SWITCH_TOP1_BF16):
        counts = _counts(spec, spec.T * spec.k)
        names = ["route", "gemm1_act", "gemm2"] + (["gemm1_act_shared", "gemm2_shared"] if spec.F_shared else [])
        total = sum(bench.kernel_work(spec, counts, n)[0] for n in names)
        assert abs(total - bench.active_flops(spec, counts)) <= 1e-9 * total


def test_bound_follows_arithmetic_intensity():
    pre, dec = workloads.MIXTRAL_PREFILL_BF16, workloads.MIXTRAL_DECODE_BF16
    fl, nb = bench.kernel_work(pre, _counts(pre, 8192), "gemm1_act")
    assert abs(fl - 2 * 8192 * 4096 * 14336 * 2) < 1
    # routed rows + gate/up weights of 8 experts + hidden rows, bf16
    assert abs(nb - 2 * (8192 * 4096 + 8 * 2 * 14336 * 4096 + 8192 * 14336)) < 1
    assert bench.kernel_roofline(pre, fl, nb, 1e-3)[0] == "mfma"
    fl, nb = bench.kernel_work(dec, _counts(dec, 32), "gemm1_act")
    bound, ach, peak, unit = bench.kernel_roofline(dec, fl, nb, 1e-3)
    assert (bound, unit, peak) == ("hbm", "GB/s", bench.PEAK_HBM_GBS)
    assert abs(ach - nb / 1e-3 / 1e9) < 1e-6
    scan = bench.kernel_work(pre, _counts(pre, 8192), "permute_scan")
    assert bench.kernel_roofline(pre, *scan, 1e-5)[0] == "latency"
    comb = bench.kernel_work(pre, _counts(pre, 8192), "combine")
    assert bench.kernel_roofline(pre, *comb, 1e-5)[0] == "hbm"
