"""Whole input domains against the oracle (needs an MI355X).

* bf16: every one of the 65,536 bf16 patterns as the gate (non-finite
  patterns are run but not compared), with up and dy set to 1 and to random
  values: forward and backward within 2 bf16 ulp.
* fp32: the 400,001 consecutive fp32 values centred on the minimiser
  g0 = -1 - W(1/e) of silu, where 1 + g(1 - sigma(g)) has its root and a
  direct fp32 evaluation loses every digit: all outputs within 1e-5 relative.
* fp32: a dense sweep of g over [-80, 80] and over [-140, -80] (where
  sigma(g) ~ e^g falls below the normal fp32 range at g ~ -87.3 and the
  outputs follow at g ~ -91.8), plus wide magnitudes. The relative bar
  applies wherever the reference is a normal fp32 number (|ref| >= 2^-126);
  where it is an fp32 subnormal, the same bar plus one subnormal step for
  the one rounding into that range: |got - ref| <= 1e-5 |ref| + 2^-149.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import swiglu_activation_amd as sw
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run(x_h, dy_h, dtype):
    x, dy = gu.to_dev(x_h, dtype), gu.to_dev(dy_h, dtype)
    y = sw.swiglu_gateup_fwd(x)
    dx = sw.swiglu_gateup_bwd(dy, x)
    x2 = x.clone()
    sw.swiglu_gateup_bwd(dy, x2, in_place=True)
    torch.cuda.synchronize()
    assert gu.bits_equal(x2, dx)
    return gu.from_dev(y), gu.from_dev(dx)


def _report(stats):
    for s in stats:
        print("   ", s, flush=True)
    assert all(s.ok() for s in stats), "\n".join(map(str, stats))


@pytest.mark.parametrize("companions", ["ones", "random"])
def test_bf16_every_gate_value(companions):
    print(f"[exhaustive bf16] companions={companions}", flush=True)
    rows, n = 256, 256
    g_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(rows, n)
    if companions == "ones":
        u_bits = np.full((rows, n), 0x3F80, np.uint16)
        dy_bits = np.full((rows, n), 0x3F80, np.uint16)
    else:
        rng = np.random.default_rng(21)
        u_bits = oracle.round_f64_to_bf16_bits(rng.standard_normal((rows, n)))
        dy_bits = oracle.round_f64_to_bf16_bits(rng.standard_normal((rows, n)))
    x_bits = np.concatenate([g_bits, u_bits], axis=1)
    y, dx = _run(x_bits, dy_bits, "bf16")
    xf = oracle.widen(x_bits, "bf16")
    dyf = oracle.widen(dy_bits, "bf16")
    fin = np.isfinite(oracle.widen(g_bits, "bf16"))
    with np.errstate(all="ignore"):
        yref = oracle.oracle_fwd(xf)
        dref = oracle.oracle_bwd(xf, dyf)
    ok_y = fin & ~np.isnan(yref)          # every finite gate
    _report([gu.compare(y, yref, "bf16", "fwd", mask=ok_y),
             gu.compare(dx[:, :n], dref[:, :n], "bf16", "dgate", mask=fin & ~np.isnan(dref[:, :n])),
             gu.compare(dx[:, n:], dref[:, n:], "bf16", "dup", mask=fin & ~np.isnan(dref[:, n:]))])


@pytest.mark.parametrize("companions", ["ones", "random"])
def test_fp32_neighbourhood_of_silu_minimiser(companions):
    print(f"[exhaustive fp32 near g0] companions={companions}", flush=True)
    center = np.float32(oracle.G0).view(np.int32).astype(np.int64)
    cnt = 400_001
    n = 4096
    rows = -(-cnt // n)
    # consecutive patterns of negative floats: larger pattern = more negative
    pats = center - 200_000 + np.arange(rows * n, dtype=np.int64)
    g = pats.astype(np.int32).view(np.float32).reshape(rows, n)
    if companions == "ones":
        u = np.ones((rows, n), np.float32)
        dy = np.ones((rows, n), np.float32)
    else:
        rng = np.random.default_rng(22)
        u = rng.standard_normal((rows, n)).astype(np.float32)
        dy = rng.standard_normal((rows, n)).astype(np.float32)
    x = np.concatenate([g, u], axis=1)
    y, dx = _run(x, dy, "fp32")
    xf, dyf = x.astype(np.float64), dy.astype(np.float64)
    yref, dref = oracle.oracle_fwd(xf), oracle.oracle_bwd(xf, dyf)
    _report([gu.compare(y, yref, "fp32", "fwd"),
             gu.compare(dx[:, :n], dref[:, :n], "fp32", "dgate"),
             gu.compare(dx[:, n:], dref[:, n:], "fp32", "dup")])


def test_fp32_sweep():
    print("[fp32 sweep]", flush=True)
    rng = np.random.default_rng(23)
    n = 4096
    g = np.concatenate([
        np.linspace(-80.0, 80.0, 1 << 20),
        np.linspace(-140.0, -80.0, 1 << 18),
        rng.uniform(-30, 30, 1 << 19),
        np.ldexp(rng.uniform(1, 2, 1 << 17), rng.integers(-100, 100, 1 << 17))
        * rng.choice([-1.0, 1.0], 1 << 17),
        [0.0, -0.0, 1e-30, -1e-30, 88.0, -87.0, 1e30],
    ])
    rows = -(-g.size // n)
    g = np.concatenate([g, np.zeros(rows * n - g.size)]).astype(np.float32).reshape(rows, n)
    u = rng.standard_normal((rows, n)).astype(np.float32)
    dy = rng.standard_normal((rows, n)).astype(np.float32)
    x = np.concatenate([g, u], axis=1)
    y, dx = _run(x, dy, "fp32")
    xf, dyf = x.astype(np.float64), dy.astype(np.float64)
    with np.errstate(all="ignore"):
        yref, dref = oracle.oracle_fwd(xf), oracle.oracle_bwd(xf, dyf)
    tiny = 2.0 ** -126
    big = np.finfo(np.float32).max

    def normal(r):
        return (np.abs(r) >= tiny) & (np.abs(r) <= big) | (r == 0)

    _report([gu.compare(y, yref, "fp32", "fwd", mask=normal(yref)),
             gu.compare(dx[:, :n], dref[:, :n], "fp32", "dgate", mask=normal(dref[:, :n])),
             gu.compare(dx[:, n:], dref[:, n:], "fp32", "dup", mask=normal(dref[:, n:]))])
    # subnormal references: the relative bar plus one subnormal step
    for got, ref, what in ((y, yref, "fwd"), (dx[:, :n], dref[:, :n], "dgate"),
                           (dx[:, n:], dref[:, n:], "dup")):
        sub = (np.abs(ref) < tiny) & (ref != 0)
        err = np.abs(got.astype(np.float64)[sub] - ref[sub]) - 1e-5 * np.abs(ref[sub])
        worst = float(err.max() / 2.0 ** -149) if err.size else 0.0
        print(f"    {what}: {int(sub.sum())} subnormal references, worst excess over 1e-5 |ref| "
              f"{worst:.3g} steps", flush=True)
        assert sub.sum() > 0 and worst <= 1.0, (what, worst)
