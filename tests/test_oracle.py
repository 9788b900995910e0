"""The CPU oracle against mathematics, libraries and brute force (no GPU)."""

from __future__ import annotations

import json
import math
import os
import types
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import oracle_pins as pins

HERE = os.path.dirname(os.path.abspath(__file__))


def _impl(**over):
    base = dict(sigmoid=oracle.sigmoid, silu=oracle.silu, silu_grad=oracle.silu_grad,
                oracle_fwd=oracle.oracle_fwd, oracle_bwd=oracle.oracle_bwd,
                oracle_fwd_bias_scale=oracle.oracle_fwd_bias_scale,
                oracle_bwd_bias_scale=oracle.oracle_bwd_bias_scale,
                oracle_fc1=oracle.oracle_fc1, oracle_fc1_swiglu=oracle.oracle_fc1_swiglu)
    base.update(over)
    return types.SimpleNamespace(**base)


def _tiny_inputs():
    w = synth.WORKLOADS[synth.SMALL]
    x = oracle.widen(synth.make_x(w), w.dtype)
    dy = oracle.widen(synth.make_dy(w), w.dtype)
    return x, dy


# --------------------------------------------------------------------------
# The oracle passes every pin
# --------------------------------------------------------------------------

@pytest.mark.parametrize("pin", pins.ALL_PINS + pins.BIAS_SCALE_PINS + pins.FC1_PINS,
                         ids=lambda p: p.__name__)
def test_pin(pin):
    pin(_impl())


def test_g0_constant_matches_lambert_w():
    assert abs(oracle.G0 - pins.g0_from_lambert_w()) < 4e-16


def test_finite_differences_on_tiny_workload():
    x, dy = _tiny_inputs()
    pins.pin_finite_differences(_impl(), x, dy)


def test_finite_differences_wide_range():
    rng = np.random.default_rng(11)
    g = np.concatenate([rng.uniform(-30, 30, 200), rng.standard_normal(200),
                        oracle.G0 + rng.uniform(-1e-3, 1e-3, 56)])
    u = rng.standard_normal(g.size) * 2
    x = np.concatenate([g, u])[None, :]
    dy = rng.standard_normal((1, g.size))
    pins.pin_finite_differences(_impl(), x, dy)


def test_high_precision_near_root():
    """fp64 oracle accuracy at the float32 points nearest g0 (the worst case
    for cancellation in 1 + g(1 - sigma))."""
    import mpmath
    g0f = np.float32(oracle.G0)
    pts = [np.nextafter(g0f, np.float32(-2)), g0f, np.nextafter(g0f, np.float32(0))]
    with mpmath.workdps(50):
        for p in pts:
            z = mpmath.mpf(float(p))
            ref = float(mpmath.diff(lambda t: t / (1 + mpmath.exp(-t)), z))
            got = oracle.silu_grad(np.array([float(p)]))[0]
            assert abs(got - ref) <= 1e-8 * abs(ref), (p, got, ref)


def test_in_place_and_3d_shapes_flatten():
    x, dy = _tiny_inputs()
    x3 = x.reshape(16, 4, 256)
    assert np.array_equal(oracle.oracle_fwd(x3), oracle.oracle_fwd(x))
    assert np.array_equal(oracle.oracle_bwd(x3, dy.reshape(16, 4, 128)), oracle.oracle_bwd(x, dy))
    with pytest.raises(ValueError):
        oracle.oracle_fwd(np.zeros((2, 3)))


# --------------------------------------------------------------------------
# Planted mistakes: each one trips at least one pin
# --------------------------------------------------------------------------

def _bwd_from(dgate_fn, dup_fn):
    def bwd(x, dy):
        g, u = oracle.split_gate_up(x)
        dy = np.asarray(dy, np.float64).reshape(g.shape)
        s = 1.0 / (1.0 + np.exp(-g))
        return np.concatenate([dgate_fn(g, u, dy, s), dup_fn(g, u, dy, s)], axis=1)
    return bwd


def _ok_dgate(g, u, dy, s):
    return dy * u * s * (1 + g * (1 - s))


def _ok_dup(g, u, dy, s):
    return dy * g * s


def _fwd_swapped(x):
    g, u = oracle.split_gate_up(x)
    return oracle.silu(u) * g


MUTANTS = {
    "halves_swapped_fwd": dict(oracle_fwd=_fwd_swapped),
    "dropped_one_in_grad": dict(
        silu_grad=lambda z: oracle.sigmoid(z) * (z * (1 - oracle.sigmoid(z))),
        oracle_bwd=_bwd_from(lambda g, u, dy, s: dy * u * s * (g * (1 - s)), _ok_dup)),
    "sign_flip_in_grad": dict(
        silu_grad=lambda z: oracle.sigmoid(z) * (1 + z * oracle.sigmoid(z)),
        oracle_bwd=_bwd_from(lambda g, u, dy, s: dy * u * s * (1 + g * s), _ok_dup)),
    "dgate_missing_up": dict(
        oracle_bwd=_bwd_from(lambda g, u, dy, s: dy * s * (1 + g * (1 - s)), _ok_dup)),
    "dup_missing_dy": dict(oracle_bwd=_bwd_from(_ok_dgate, lambda g, u, dy, s: g * s)),
    "dgate_dup_swapped": dict(oracle_bwd=_bwd_from(_ok_dup, _ok_dgate)),
    "sigmoid_wrong_sign": dict(sigmoid=lambda z: 1.0 / (1.0 + np.exp(np.asarray(z, float)))),
    "silu_is_sigmoid": dict(silu=lambda z: oracle.sigmoid(z)),
    "grad_is_sigmoid": dict(silu_grad=lambda z: oracle.sigmoid(z)),
    "fwd_missing_up": dict(oracle_fwd=lambda x: oracle.silu(oracle.split_gate_up(x)[0])),
}


def _bs_bwd_mutant(kind):
    def bwd(x, dy, bias=None, scale=None):
        dx, db, ds = oracle.oracle_bwd_bias_scale(x, dy, bias, scale)
        x2 = np.asarray(x, float).reshape(np.asarray(dy).shape[0], -1)
        z = x2 + (0 if bias is None else np.asarray(bias, float))
        if kind == "dscale_without_up" and scale is not None:
            n = z.shape[1] // 2
            ds = (np.asarray(dy, float) * oracle.silu(z[:, :n])).sum(axis=1)
        if kind == "dbias_from_unscaled" and bias is not None:
            db = oracle.oracle_bwd(z, dy).sum(axis=0)
        if kind == "dx_unscaled":
            dx = oracle.oracle_bwd(z, dy)
        return dx, db, ds
    return bwd


def _fwd_scale_inside_silu(x, b=None, s=None):
    z = np.asarray(x, float) + (0.0 if b is None else np.asarray(b, float))
    if s is not None:
        n = z.shape[1] // 2
        z = z.copy()
        z[:, :n] *= np.asarray(s, float)[:, None]
    return oracle.oracle_fwd(z)


BS_MUTANTS = {
    "bias_ignored": dict(oracle_fwd_bias_scale=lambda x, b=None, s=None:
                         oracle.oracle_fwd_bias_scale(x, None, s)),
    "scale_inside_silu": dict(oracle_fwd_bias_scale=_fwd_scale_inside_silu),
    "dscale_without_up": dict(oracle_bwd_bias_scale=_bs_bwd_mutant("dscale_without_up")),
    "dbias_from_unscaled": dict(oracle_bwd_bias_scale=_bs_bwd_mutant("dbias_from_unscaled")),
    "dx_unscaled": dict(oracle_bwd_bias_scale=_bs_bwd_mutant("dx_unscaled")),
}


@pytest.mark.parametrize("name", sorted(BS_MUTANTS))
def test_planted_bias_scale_mistake_is_caught(name):
    impl = _impl(**BS_MUTANTS[name])
    caught = 0
    for pin in pins.BIAS_SCALE_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"mutant {name} passed every pin"


FC1_MUTANTS = {
    "fc1_reshape_for_transpose": dict(oracle_fc1=lambda a, w: np.asarray(a, float) @ np.asarray(
        w, float).reshape(np.asarray(w).shape[1], np.asarray(w).shape[0])),
    "fc1_halves_swapped": dict(oracle_fc1_swiglu=lambda a, w: oracle.oracle_fwd(
        oracle.oracle_fc1(a, np.concatenate([np.asarray(w)[np.asarray(w).shape[0] // 2:],
                                             np.asarray(w)[:np.asarray(w).shape[0] // 2]])))),
    "fc1_sum_off_by_one": dict(oracle_fc1=lambda a, w: np.asarray(a, float)[:, 1:] @ np.asarray(w, float)[:, 1:].T),
}


@pytest.mark.parametrize("name", sorted(FC1_MUTANTS))
def test_planted_fc1_mistake_is_caught(name):
    impl = _impl(**FC1_MUTANTS[name])
    caught = 0
    for pin in pins.FC1_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, TypeError, ValueError):
            caught += 1
    assert caught >= 1, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    impl = _impl(**MUTANTS[name])
    x, dy = _tiny_inputs()
    checks = list(pins.ALL_PINS) + [lambda i: pins.pin_finite_differences(i, x, dy)]
    caught = 0
    for pin in checks:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"mutant {name} passed every pin"


# --------------------------------------------------------------------------
# bf16 rounding and ulp distance
# --------------------------------------------------------------------------

def _nearest_bf16_bruteforce(v: float) -> int:
    """Exact nearest bf16 (ties to even) by rational arithmetic over the
    ordered list of all finite bf16 values near v."""
    if v != v:
        raise ValueError
    fv = Fraction(v)
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = abs(fv)
    maxv = Fraction(255, 1) * Fraction(2) ** 120
    if a >= maxv + Fraction(2) ** 119:    # at or past the midpoint to 2^128
        return sign | 0x7F80
    # candidate magnitudes: all bf16 patterns whose value brackets a
    best, best_d = None, None
    lo, hi = 0, 0x7F7F
    while lo < hi:                      # largest pattern with value <= a
        mid = (lo + hi + 1) // 2
        if _bf16_frac(mid) <= a:
            lo = mid
        else:
            hi = mid - 1
    for m in (lo, min(lo + 1, 0x7F7F)):
        d = abs(_bf16_frac(m) - a)
        if best is None or d < best_d or (d == best_d and (m & 1) == 0):
            best, best_d = m, d
    return sign | best


def _bf16_frac(m: int) -> Fraction:
    e = (m >> 7) & 0xFF
    f = m & 0x7F
    if e == 0:
        return Fraction(f) * Fraction(2) ** -133
    return Fraction(128 + f) * Fraction(2) ** (e - 134)


def test_bf16_rounding_bruteforce():
    rng = np.random.default_rng(3)
    vals = list(rng.standard_normal(300))
    vals += list(np.ldexp(rng.uniform(1, 2, 300), rng.integers(-140, 128, 300)))
    # exact ties and near-ties between consecutive bf16 values
    for m in rng.integers(1, 0x7F7F, 200):
        a, b = float(_bf16_frac(int(m))), float(_bf16_frac(int(m) + 1))
        mid = (a + b) / 2
        vals += [mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf)]
    vals += [0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134, 2.0 ** -150,
             1 + 2 ** -8 + 2 ** -30, 255.5 * 2.0 ** 120, np.nextafter(255.5 * 2.0 ** 120, 0),
             1e300, -1e-300]
    vals = [float(v) * s for v in vals for s in (1.0, -1.0)]
    got = oracle.round_f64_to_bf16_bits(np.array(vals))
    for v, b in zip(vals, got):
        assert int(b) == _nearest_bf16_bruteforce(v), (v, hex(int(b)))


def test_bf16_rounding_matches_torch_on_float32_values():
    """For values that are exact in float32, one direct rounding equals
    torch's float32 -> bfloat16 conversion (round to nearest even)."""
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    f32 = bits.view(np.float32)
    f32 = f32[np.isfinite(f32)]
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_f64_to_bf16_bits(f32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_no_double_rounding():
    v = 1 + 2 ** -8 + 2 ** -30      # above the 1 / 1+2^-7 midpoint, but float32 rounds it onto it
    assert np.float32(v) == np.float32(1 + 2 ** -8)
    assert int(oracle.round_f64_to_bf16_bits(np.array([v]))[0]) == 0x3F81


def test_bf16_widen_exact():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_bits_to_f64(allbits)
    fin = np.isfinite(v)
    back = oracle.round_f64_to_bf16_bits(v[fin])
    assert np.array_equal(back, allbits[fin])
    assert oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0001], np.uint16)).tolist() == \
        [1.0, -2.0, 2.0 ** -133]


def test_bf16_ulp_distance():
    d = oracle.bf16_ulp_distance
    u16 = lambda *a: np.array(a, np.uint16)  # noqa: E731
    assert d(u16(0x0000), u16(0x8000))[0] == 0
    assert d(u16(0x0001), u16(0x8001))[0] == 2
    assert d(u16(0x3F80), u16(0x3F7F))[0] == 1           # across a binade edge
    assert d(u16(0x7F7F), u16(0x7F80))[0] == 1           # max finite to inf
    assert d(u16(0xBF80), u16(0x3F80))[0] == 2 * 0x3F80
    # monotone: the ordinal sorts all finite bf16 values like their values do
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_bits_to_f64(allbits)
    fin = np.isfinite(v)
    o = oracle.bf16_ordinal(allbits[fin])
    order = np.argsort(v[fin], kind="stable")
    assert np.all(np.diff(o[order]) >= 0)


def _is_nearest_bf16(v: Fraction, bits: int) -> bool:
    """bits is a nearest (ties to even) bf16 of the exact value v; a result
    of zero may carry either sign."""
    m = bits & 0x7FFF
    if m == 0:
        return abs(v) <= Fraction(2) ** -134        # half the smallest subnormal (a tie goes to 0)
    if v == 0 or (v < 0) != bool(bits & 0x8000):
        return False
    a = abs(v)
    if m == 0x7F80:
        return a >= Fraction(255) * Fraction(2) ** 120 + Fraction(2) ** 119
    d = abs(_bf16_frac(m) - a)
    for nb in (m - 1, m + 1):
        if 0 <= nb <= 0x7F7F:
            dn = abs(_bf16_frac(nb) - a)
            if dn < d or (dn == d and nb % 2 == 0):
                return False
    return True


def _mp_to_fraction(x) -> Fraction:
    sign, man, exp, _ = x._mpf_                          # value = (-1)^sign * man * 2^exp
    return (-1 if sign else 1) * Fraction(int(man)) * Fraction(2) ** int(exp)


def test_bf16_rounding_of_oracle_equals_50_digit_rounding_on_every_gate():
    """For every finite bf16 gate value g, the oracle's float64 silu(g) and
    silu'(g) (the forward and dgate with u = dy = 1), rounded once to bf16,
    are the nearest bf16 values of the 50-digit results. The derivative is
    taken by the quotient rule, 1/(1+e^-g) + g e^-g / (1+e^-g)^2, not in the
    oracle's form.

    One exception, asserted exactly: for a gate below 2^-125 in magnitude
    with an odd last bit, silu(g) = g/2 + g^2/4 + ... where float64 keeps
    only g/2, a bf16 subnormal plus exactly half a step; the oracle rounds
    that tie to even, the exact value lies just past it. Those forwards
    differ by one subnormal step (2^-133)."""
    import mpmath
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g = oracle.bf16_bits_to_f64(allbits)
    g = g[np.isfinite(g)]
    y_bits = oracle.round_f64_to_bf16_bits(oracle.silu(g))
    d_bits = oracle.round_f64_to_bf16_bits(oracle.silu_grad(g))
    tiny = mpmath.mpf(2) ** -140
    bad = []
    with mpmath.workdps(50):
        for gv, yb, db in zip(g.tolist(), y_bits.tolist(), d_bits.tolist()):
            G = mpmath.mpf(gv)
            e = mpmath.exp(-G)
            silu = G / (1 + e)
            grad = 1 / (1 + e) + G * e / (1 + e) ** 2
            for val, bits in ((silu, yb), (grad, db)):
                if abs(val) < tiny:
                    ok = (bits & 0x7FFF) == 0
                else:
                    ok = _is_nearest_bf16(_mp_to_fraction(val), int(bits))
                if not ok:
                    bad.append((gv, val is silu, int(bits)))
    tie_cases = 0
    for gv, is_fwd, bits in bad:
        # only forwards at gates whose half is subnormal and whose float64 value is an exact tie
        assert is_fwd and 0 < abs(gv) < 2.0 ** -125, (gv, is_fwd, hex(bits))
        y64 = float(oracle.silu(np.array([gv]))[0])
        assert y64 == gv / 2
        scaled = abs(y64) * 2.0 ** 133                  # in units of the smallest subnormal
        assert scaled % 1 == 0.5, (gv, scaled)
        tie_cases += 1
    odd_tiny = int(np.sum((np.abs(g) < 2.0 ** -125) & (g != 0) &
                          (oracle.round_f64_to_bf16_bits(np.abs(g)) % 2 == 1)))
    assert tie_cases <= odd_tiny == 256
    print(f"{tie_cases} tie cases of {g.size} gates")


def test_minimiser_identities():
    """At g0: sigma(g0) = 1 + 1/g0 (silu'(g0) = 0 solved for sigma), and the
    bracket h(g) = silu'(g) / sigma(g) = 1 + g (1 - sigma(g)) crosses zero
    with slope exactly 1 (h' = (1 - sigma)(1 - g sigma) = (-1/g0)(-g0))."""
    g0 = oracle.G0
    assert abs(oracle.sigmoid(np.array([g0]))[0] - (1 + 1 / g0)) < 1e-15
    d = 1e-6
    gs = np.array([g0 - d, g0 + d])
    h = oracle.silu_grad(gs) / oracle.sigmoid(gs)
    assert abs((h[1] - h[0]) / (2 * d) - 1.0) < 1e-8


# --------------------------------------------------------------------------
# Golden fixture (written by tests/golden/make_golden.py from the oracle)
# --------------------------------------------------------------------------

def test_golden_fixture_regression():
    with open(os.path.join(HERE, "golden", "swiglu_small.json")) as f:
        gold = json.load(f)
    x = np.array([[float.fromhex(v) for v in row] for row in gold["x"]])
    dy = np.array([[float.fromhex(v) for v in row] for row in gold["dy"]])
    y = oracle.oracle_fwd(x)
    dx = oracle.oracle_bwd(x, dy)
    y_ref = np.array([[float.fromhex(v) for v in row] for row in gold["y"]])
    dx_ref = np.array([[float.fromhex(v) for v in row] for row in gold["dx"]])
    assert np.array_equal(y, y_ref)
    assert np.array_equal(dx, dx_ref)
    assert oracle.round_f64_to_bf16_bits(y).tolist() == gold["y_bf16_bits"]
    assert oracle.round_f64_to_bf16_bits(dx).tolist() == gold["dx_bf16_bits"]
