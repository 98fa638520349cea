"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each exercised by the CPU tests that load it, in a subprocess
with the sanitizer runtime preloaded:
  * the oracle (plain C) built by gcc with -fsanitize=address,undefined, run
    through every oracle pin;
  * the HIP library with its host code (argument checks, configuration
    derivation, workspace carving, launch set-up) built with the same
    sanitizers on the host pass only, run through the C-ABI host tests.
A run passes only if the tests pass and the sanitizers write no report.
GPU code is not sanitized (no device sanitizer is used here).
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _run(tmp_path, env_extra, tests):
    logs = tmp_path / "san"
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:log_path={logs}"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={logs}"
    env.setdefault("OMP_NUM_THREADS", "4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = sorted(glob.glob(str(logs) + "*"))
    text = "".join(open(f).read() for f in reports)
    assert r.returncode == 0 and not reports, f"rc={r.returncode}\n{r.stdout[-3000:]}\n{text[:6000]}"
    return r.stdout


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan(tmp_path):
    import oracle
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_sanitized.so"))
    out = _run(tmp_path, {"LD_PRELOAD": f"{asan}:{ubsan}", "ORACLE_LIB": lib},
               ["tests/test_oracle_pins.py"])
    assert " passed" in out


def test_library_host_code_under_asan_ubsan(tmp_path):
    from sparse_mixture_experts_gating_amd import build
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build(sanitize=True)
    out = _run(tmp_path, {"LD_PRELOAD": runtime, "MOE_HIP_LIB": lib},
               ["tests/test_boundary_host.py", "tests/test_bench_host.py"])
    assert " passed" in out
