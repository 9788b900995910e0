"""bench.py's host-side contract, on the CPU: the one-GPU refusal, the exit
without a GPU, the roofline object and the oracle timing legs."""
import os
import subprocess
import sys
import types

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2", "--steps", "3", "--warmup", "1")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the exit without a GPU")
def test_exits_without_a_gpu():
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr and r.stdout == ""


def test_hbm_roofline_object():
    r = bench.hbm_roofline("k", 4.0e9, 0.5)          # 4 GB in 0.5 ms = 8000 GB/s
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_GBPS
    assert r["achieved"] == pytest.approx(8000.0) and r["frac"] == pytest.approx(1.0)
    assert r["bytes_per_launch"] == 4.0e9


def _small_workload(rows=64, n=256):
    rng = np.random.default_rng(0)
    # bf16 bit patterns of modest normal values: sign, exponents 120..130
    def bits(shape):
        e = rng.integers(120, 131, size=shape).astype(np.uint16)
        return ((rng.integers(0, 2, size=shape).astype(np.uint16) << 15) | (e << 7)
                | rng.integers(0, 128, size=shape).astype(np.uint16))
    w = types.SimpleNamespace(rows=rows, n=n, dtype="bf16", elem_bytes=2, name="small", seed=0)
    return w, bits((rows, 2 * n)), bits((rows, n))


def test_cpu_baseline_covers_the_sample_it_reports():
    # fewer rows than the 512 the bias / scale sample takes by default
    w, x, dy = _small_workload(rows=256, n=2048)
    r = bench.cpu_baseline(w, x, dy, seconds=30.0)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["unit"] == "GB/s"
    assert r["sample"].startswith(f"rows 0..{w.rows} of {w.rows}")
    assert r["value"] > 0 and r["seconds"] > 0
    # (seconds is reported to the millisecond)
    assert r["value"] == pytest.approx(8 * 2 * w.rows * w.n / r["seconds"] / 1e9, rel=0.05)
    a = r["all_cores"]
    assert 1 <= a["cores"] <= 16 and a["value"] > 0
    assert set(r["other_rows"]) == {"bias_scale", "fc1_swiglu"}


def test_all_cores_leg_runs_every_block():
    # a row count that is not a multiple of the block: the last block is short
    w, x, dy = _small_workload(rows=70)
    r = bench.cpu_baseline_all_cores(w, x, dy, block=32, max_threads=4)
    assert r["cores"] == min(4, len(os.sched_getaffinity(0)))
    assert f"all {w.rows} rows" in r["sample"]


def test_cpu_baseline_compares_the_timed_outputs_with_the_oracle():
    import oracle
    w, x, dy = _small_workload(rows=48, n=128)
    xf, dyf = oracle.widen(x, "bf16"), oracle.widen(dy, "bf16")
    y = oracle.round_f64_to_bf16_bits(oracle.oracle_fwd(xf))
    dx = oracle.round_f64_to_bf16_bits(oracle.oracle_bwd(xf, dyf))
    r = bench.cpu_baseline(w, x, dy, seconds=30.0, outputs=(y, dx))["timed_outputs_vs_oracle"]
    assert r == {"rows": 48, "elements": 3 * 48 * 128, "max_ulp_fwd": 0, "max_ulp_bwd": 0,
                 "over_2_ulp": 0}
    # a planted error of 3 ulp in one dgate element (away from zero and the
    # binade edges) is reported
    dx_bad = dx.copy()
    i, j = 17, 5
    dx_bad[i, j] = np.uint16(int(dx_bad[i, j]) + (3 if (dx_bad[i, j] & 0x7F) < 0x7C else -3))
    r = bench.cpu_baseline(w, x, dy, seconds=30.0, outputs=(y, dx_bad))["timed_outputs_vs_oracle"]
    assert r["max_ulp_fwd"] == 0 and r["max_ulp_bwd"] == 3 and r["over_2_ulp"] == 1
    # without outputs there is no comparison
    assert bench.cpu_baseline(w, x, dy, seconds=30.0)["timed_outputs_vs_oracle"] is None


def test_oracle_parity_counts_planted_errors():
    import oracle
    rng = np.random.default_rng(1)
    ref = rng.standard_normal(1000)
    # bf16: the correctly rounded bits, one element moved 3 steps and one 2
    bits = oracle.round_f64_to_bf16_bits(ref).copy()
    bits[10] += 3
    bits[20] += 2
    st = bench.oracle_parity("bf16", bits, ref)
    assert st == {"elements": 1000, "max_ulp": 3, "over_2_ulp": 1}
    # fp32: one element 2e-5 off in relative terms, one nonzero where ref is 0
    ref[5] = 0.0
    got = ref.astype(np.float32)
    got[7] = np.float32(ref[7] * (1 + 2e-5))
    got[5] = np.float32(1e-30)
    st = bench.oracle_parity("fp32", got, ref, den=np.abs(ref) + 1.0)
    assert st["over_1e-5"] == 2
    assert 1.5e-5 < st["max_rel"] < 2.5e-5
    assert st["max_scale_aware"] > 0


def test_oracle_parity_of_exact_sample_is_clean():
    import oracle
    import synth
    for name in ("tiny_fp32_s16_b4_n128", "inplace_tp_bf16_t8192_n1792"):
        w = synth.WORKLOADS[name]
        x, dy = synth.make_x(w, 0, 16), synth.make_dy(w, 0, 16)
        xf, dyf = oracle.widen(x, w.dtype), oracle.widen(dy, w.dtype)
        y, dx = oracle.oracle_fwd(xf), oracle.oracle_bwd(xf, dyf)
        if w.dtype == "bf16":
            y, dx = oracle.round_f64_to_bf16_bits(y), oracle.round_f64_to_bf16_bits(dx)
        else:
            y, dx = y.astype(np.float32), dx.astype(np.float32)
        st = bench.oracle_parity_of_sample(w.dtype, w.n, {"rows": [0, 16], "x": x, "dy": dy,
                                                          "y": y, "dx": dx})
        key = "over_2_ulp" if w.dtype == "bf16" else "over_1e-5"
        for p in ("fwd", "bwd_dgate", "bwd_dup"):
            assert st[p][key] == 0 and st[p]["elements"] == 16 * w.n
        # storage rounding alone: half a step of the stored type, relative
        assert st["bwd_dgate"]["max_scale_aware"] < (2.0 ** -8 if w.dtype == "bf16" else 1e-6)
