"""Pins of the CPU oracle against things other than itself.

Each pin takes an implementation namespace ``impl`` with the oracle's
functions (sigmoid, silu, silu_grad, oracle_fwd, oracle_bwd) and raises
AssertionError when the implementation disagrees with mathematics or a
library routine. ``tests/test_oracle.py`` runs every pin on the oracle (all
must pass) and on planted mistakes (each must trip at least one pin).

What pins what:
* closed forms: silu(0) = 0, sigma(0) = 1/2, silu'(0) = 1/2, silu''(0) = 1/2,
  silu(x) = x in float64 for x >= 37, silu(x) -> x*exp(x) -> 0- for x -> -inf;
* a library routine: sigma against scipy.special.expit (the logistic function);
* the minimiser: silu' changes sign at g0 = -1 - W(1/e) (scipy's Lambert W),
  silu(g0) = 1 + g0 and silu is smallest there;
* identities: silu(x) - silu(-x) = x and silu'(x) + silu'(-x) = 1;
* derivative: mpmath's numerical differentiation of z / (1 + exp(-z)) at 40
  digits, and central finite differences of the forward for the backward;
* layout: which half is the gate, which is the up half, and where the
  backward writes dgate and dup.
"""

from __future__ import annotations

import math

import mpmath
import numpy as np
import scipy.special


def g0_from_lambert_w() -> float:
    return float(-1.0 - scipy.special.lambertw(math.exp(-1.0)).real)


def pin_closed_forms(impl):
    assert impl.silu(np.array([0.0]))[0] == 0.0
    assert impl.sigmoid(np.array([0.0]))[0] == 0.5
    assert abs(impl.silu_grad(np.array([0.0]))[0] - 0.5) < 1e-15
    h = 1e-4
    d2 = (impl.silu_grad(np.array([h]))[0] - impl.silu_grad(np.array([-h]))[0]) / (2 * h)
    assert abs(d2 - 0.5) < 1e-8, d2
    big = np.array([37.0, 40.0, 100.0, 1e3, 1e10])
    assert np.array_equal(impl.silu(big), big)
    for x in (-20.0, -40.0, -100.0, -700.0):
        ref = x * math.exp(x) / (1.0 + math.exp(x))
        got = impl.silu(np.array([x]))[0]
        assert got < 0.0 and abs(got - ref) <= 1e-14 * abs(ref), (x, got, ref)
    with np.errstate(all="ignore"):
        vneg = impl.silu(np.array([-800.0, -1e30]))
    assert np.all(vneg == 0.0)


def pin_expit(impl):
    z = np.concatenate([np.linspace(-40, 40, 4001), [-700.0, -300.0, 300.0, 700.0]])
    ref = scipy.special.expit(z)
    got = impl.sigmoid(z)
    assert np.all(np.abs(got - ref) <= 4e-16 * np.abs(ref) + 1e-300)


def pin_minimiser(impl):
    g0 = g0_from_lambert_w()
    d = 1e-7
    lo, hi = impl.silu_grad(np.array([g0 - d, g0 + d]))
    assert lo < 0.0 < hi, (lo, hi)
    at = impl.silu_grad(np.array([g0]))[0]
    assert abs(at) < 1e-15, at
    assert abs(impl.silu(np.array([g0]))[0] - (1.0 + g0)) < 1e-15
    vals = impl.silu(np.array([g0 - 1e-3, g0, g0 + 1e-3]))
    assert vals[1] < vals[0] and vals[1] < vals[2]


def pin_symmetry(impl):
    x = np.linspace(-40.0, 40.0, 8001)
    assert np.max(np.abs(impl.silu(x) - impl.silu(-x) - x)) < 1e-13
    assert np.max(np.abs(impl.silu_grad(x) + impl.silu_grad(-x) - 1.0)) < 1e-14


def pin_mpmath_derivative(impl):
    """silu' against 40-digit numerical differentiation of the definition."""
    rng = np.random.default_rng(7)
    pts = np.concatenate([rng.uniform(-30, 30, 24), [-5.0, -1.0, -0.25, 0.0, 0.3, 2.0, 9.0]])
    with mpmath.workdps(40):
        for z in pts:
            ref = float(mpmath.diff(lambda t: t / (1 + mpmath.exp(-t)), mpmath.mpf(float(z))))
            got = impl.silu_grad(np.array([z]))[0]
            assert abs(got - ref) <= 1e-14 * max(1.0, abs(ref)), (z, got, ref)


def pin_finite_differences(impl, x, dy):
    """Backward of the oracle against central differences of its forward."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    n = x.shape[1] // 2
    dx = impl.oracle_bwd(x, dy)
    for half in (0, 1):
        cols = slice(half * n, (half + 1) * n)
        step = 2.0 ** -18 * np.maximum(1.0, np.abs(x[:, cols]))
        xp, xm = x.copy(), x.copy()
        xp[:, cols] += step
        xm[:, cols] -= step
        hstep = (xp[:, cols] - xm[:, cols])  # the step actually taken
        fd = dy * (impl.oracle_fwd(xp) - impl.oracle_fwd(xm)) / hstep
        g, u = x[:, :n], x[:, n:]
        tol = 1e-8 * (1.0 + np.abs(dy) * (np.abs(u) + np.abs(g) + 1.0))
        err = np.abs(fd - dx[:, cols])
        assert np.all(err <= tol), (half, float(np.max(err / tol)))


def pin_layout(impl):
    """Gate is the first half, up the second; dx is [dgate | dup]."""
    x = np.array([[100.0, 0.0, 0.5, 3.0]])     # n = 2: g = [100, 0], u = [0.5, 3]
    y = impl.oracle_fwd(x)
    assert y.shape == (1, 2)
    assert abs(y[0, 0] - 50.0) < 1e-12       # silu(100) * 0.5 = 50
    assert y[0, 1] == 0.0                    # silu(0) * 3 = 0
    dy = np.array([[2.0, 1.0]])
    dx = impl.oracle_bwd(x, dy)
    assert dx.shape == (1, 4)
    assert abs(dx[0, 0] - 2.0 * 0.5 * 1.0) < 1e-12    # dgate at g=100: silu' = 1
    assert abs(dx[0, 1] - 1.0 * 3.0 * 0.5) < 1e-15    # dgate at g=0: silu' = 1/2
    assert abs(dx[0, 2] - 2.0 * 100.0) < 1e-12        # dup = dy * silu(100)
    assert dx[0, 3] == 0.0                            # dup = dy * silu(0)


ALL_PINS = [pin_closed_forms, pin_expit, pin_minimiser, pin_symmetry,
            pin_mpmath_derivative, pin_layout]


def pin_bias_scale_reduces_to_base(impl):
    """With bias = 0 and scale = 1 the variants are the base op, and a bias
    is the same as adding it to x first."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((5, 12)) * 2
    dy = rng.standard_normal((5, 6))
    assert np.array_equal(impl.oracle_fwd_bias_scale(x), impl.oracle_fwd(x))
    dx, db, ds = impl.oracle_bwd_bias_scale(x, dy)
    assert db is None and ds is None and np.array_equal(dx, impl.oracle_bwd(x, dy))
    y1 = impl.oracle_fwd_bias_scale(x, np.zeros(12), np.ones(5))
    assert np.max(np.abs(y1 - impl.oracle_fwd(x))) == 0.0
    b = rng.standard_normal(12)
    assert np.array_equal(impl.oracle_fwd_bias_scale(x, b), impl.oracle_fwd(x + b))


def pin_bias_scale_finite_differences(impl):
    """dx, dbias and dscale against central differences of the forward in
    x, bias and scale (the loss is sum(dy * y))."""
    rng = np.random.default_rng(32)
    rows, n = 4, 5
    x = rng.standard_normal((rows, 2 * n)) * 2
    b = rng.standard_normal(2 * n)
    s = rng.uniform(0.2, 2.0, rows)
    dy = rng.standard_normal((rows, n))
    dx, db, ds = impl.oracle_bwd_bias_scale(x, dy, b, s)

    def loss(xx, bb, ss):
        return float(np.sum(dy * impl.oracle_fwd_bias_scale(xx, bb, ss)))

    h = 1e-6
    for idx in np.ndindex(x.shape):
        e = np.zeros_like(x)
        e[idx] = h
        fd = (loss(x + e, b, s) - loss(x - e, b, s)) / (2 * h)
        assert abs(fd - dx[idx]) <= 1e-6 * (1 + abs(fd)), ("dx", idx, fd, dx[idx])
    for k in range(2 * n):
        e = np.zeros_like(b)
        e[k] = h
        fd = (loss(x, b + e, s) - loss(x, b - e, s)) / (2 * h)
        assert abs(fd - db[k]) <= 1e-6 * (1 + abs(fd)), ("dbias", k, fd, db[k])
    for r in range(rows):
        e = np.zeros_like(s)
        e[r] = h
        fd = (loss(x, b, s + e) - loss(x, b, s - e)) / (2 * h)
        assert abs(fd - ds[r]) <= 1e-6 * (1 + abs(fd)), ("dscale", r, fd, ds[r])


BIAS_SCALE_PINS = [pin_bias_scale_reduces_to_base, pin_bias_scale_finite_differences]


def pin_fc1_matmul_bruteforce(impl):
    """x = A @ W.T against a triple loop on a tiny case (exact integers)."""
    rng = np.random.default_rng(51)
    a = rng.integers(-4, 5, (3, 5)).astype(float)
    w = rng.integers(-4, 5, (4, 5)).astype(float)
    x = impl.oracle_fc1(a, w)
    for i in range(3):
        for j in range(4):
            assert x[i, j] == sum(a[i, k] * w[j, k] for k in range(5))


def pin_fc1_swiglu_identity(impl):
    """With A = I the projection returns W.T, so the fused op is the base
    forward on the packed W.T; gate rows of W come first."""
    rng = np.random.default_rng(52)
    k, n = 6, 3
    w = rng.standard_normal((2 * n, k))
    y = impl.oracle_fc1_swiglu(np.eye(k), w)
    assert np.array_equal(y, impl.oracle_fwd(w.T))
    # swapping the gate and up halves of W changes the result
    assert not np.allclose(y, impl.oracle_fc1_swiglu(np.eye(k), np.concatenate([w[n:], w[:n]])))


def pin_fc1_swiglu_linear_in_up(impl):
    """y is linear in the up weights and in A's scale on the up side only
    through silu: doubling W_up doubles y."""
    rng = np.random.default_rng(53)
    a = rng.standard_normal((4, 8))
    w = rng.standard_normal((6, 8))
    w2 = w.copy()
    w2[3:] *= 2.0
    assert np.allclose(impl.oracle_fc1_swiglu(a, w2), 2.0 * impl.oracle_fc1_swiglu(a, w), rtol=1e-14)


FC1_PINS = [pin_fc1_matmul_bruteforce, pin_fc1_swiglu_identity, pin_fc1_swiglu_linear_in_up]
