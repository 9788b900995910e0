"""Plain float64 oracle of the fused gate-up SwiGLU (test infrastructure only).

What is computed, and where the pages fix it:

* Layout -- Liger-Kernel Megatron SwiGLU page, §Background: the fc1 output is
  one packed [tokens, 2n] tensor; the gate half is columns [0, n) and the up
  half is columns [n, 2n); the fused kernel reads both halves of a row through
  a column offset (input row stride 2n) and writes a [tokens, n] result (row
  stride n). Leading dimensions (2D [tokens, 2n] or 3D [s, b, 2n], §Megatron
  feature compatibility) are flattened into rows.
* Operation -- same page, §Background: the op is SiLU of the gate times up
  (the "SiLUMul" of Liger's existing two-tensor op). SiLU is the textbook
  sigmoid-weighted linear unit, silu(z) = z * sigma(z) with
  sigma(z) = 1 / (1 + exp(-z)).
* Backward -- same page, §What's added names a backward kernel over the same
  layout but prints no formula. It is the exact gradient of
  y = silu(g) * u: dup = dy * silu(g) and
  dgate = dy * u * silu'(g) = dy * u * sigma(g) * (1 + g * (1 - sigma(g))).
  silu is recomputed from the saved input x, nothing else is saved.
* In-place backward -- same page, §Optional in_place: the gradient
  [dgate | dup] may be written over the fc1 output buffer. The values are the
  same as out of place; only the destination differs, so the oracle has one
  backward.
* dtypes -- same page, §Megatron feature compatibility: fp32 and bf16.

Readings where the pages are silent: the SiLU and gate/up conventions above,
the derivative formula, and that every result is computed exactly (here in
float64) and rounded once to the storage type. The bf16 comparison target is
the float64 value rounded directly to bf16, nearest-even
(``round_f64_to_bf16_bits``), never through float32.

Every function here is pinned by ``tests/test_oracle.py`` against closed forms,
identities, high-precision numerical differentiation, brute force and library
rounding; none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

# Minimiser of silu: the root of silu'(g), i.e. of 1 + g + exp(g) = 0, which
# is g0 = -1 - W(1/e) with W the principal Lambert W branch. Tests re-derive
# it from scipy's lambertw and from a root search of this oracle's gradient.
G0 = -1.2784645427610738


# --------------------------------------------------------------------------
# Storage types -> float64
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values.

    A bf16 pattern is the upper half of the float32 with the same sign,
    exponent and leading mantissa bits, so the widening is exact.
    """
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):      # NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def widen(a, dtype: str) -> np.ndarray:
    """Stored tensor (float32 values or bf16 bit patterns) -> exact float64."""
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    raise ValueError(f"unsupported dtype {dtype!r}")


def split_gate_up(x: np.ndarray):
    """[..., 2n] -> (gate, up), each [rows, n]; gate is the first half."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % 2:
        raise ValueError("last dimension of x must be even (2n)")
    x2 = x.reshape(-1, x.shape[-1])
    n = x2.shape[1] // 2
    return x2[:, :n], x2[:, n:]


# --------------------------------------------------------------------------
# The method
# --------------------------------------------------------------------------

def sigmoid(z) -> np.ndarray:
    """sigma(z) = 1 / (1 + exp(-z)) in float64, as written.

    exp(-z) overflows to inf for z < -709.78, giving sigma = 0; the true value
    there is below 1e-308, which is 0 in every storage type used here.
    """
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z) -> np.ndarray:
    """silu(z) = z * sigma(z)."""
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def silu_grad(z) -> np.ndarray:
    """silu'(z) = sigma(z) * (1 + z * (1 - sigma(z)))."""
    z = np.asarray(z, dtype=np.float64)
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def oracle_fwd(x) -> np.ndarray:
    """Forward: y[r, c] = silu(x[r, c]) * x[r, n + c]; returns float64 [rows, n]."""
    g, u = split_gate_up(x)
    with np.errstate(invalid="ignore", over="ignore"):
        return silu(g) * u


def oracle_bwd(x, dy) -> np.ndarray:
    """Backward: returns dx = [dgate | dup] as float64 [rows, 2n].

    dgate = dy * u * sigma(g) * (1 + g * (1 - sigma(g)))
    dup   = dy * silu(g)
    """
    g, u = split_gate_up(x)
    dy = np.asarray(dy, dtype=np.float64).reshape(g.shape)
    s = sigmoid(g)
    with np.errstate(invalid="ignore", over="ignore"):
        dgate = dy * u * s * (1.0 + g * (1.0 - s))
        dup = dy * (g * s)
    return np.concatenate([dgate, dup], axis=1)


# --------------------------------------------------------------------------
# Bias and per-token scale variants
# --------------------------------------------------------------------------
# Liger-Kernel Megatron SwiGLU page, §Scope and §Known issues: Megatron's
# activation takes an optional bias on the fc1 output (bias_swiglu), and MoE
# routed experts use a per-token-scale-aware version (weighted_bias_swiglu,
# with per_token_scale). The page names these but gives no formula; the
# plainest reading, used here, is
#     z = x + bias          (bias of shape [2n], broadcast over rows)
#     y[r, c] = s[r] * silu(z[r, c]) * z[r, n + c]
# with bias = 0 and s = 1 when absent. Its exact gradient is
#     dz  = the base backward at z with upstream gradient s[r] * dy[r, c]
#     dx  = dz                      (the bias add is the identity in x)
#     dbias[k] = sum over r of dz[r, k]
#     ds[r]    = sum over c of dy[r, c] * silu(z[r, c]) * z[r, n + c]

def oracle_fwd_bias_scale(x, bias=None, scale=None) -> np.ndarray:
    """y = s * silu(z_gate) * z_up with z = x + bias; float64 [rows, n]."""
    x = np.asarray(x, dtype=np.float64)
    x2 = x.reshape(-1, x.shape[-1])
    z = x2 + (0.0 if bias is None else np.asarray(bias, dtype=np.float64).reshape(1, -1))
    y = oracle_fwd(z)
    if scale is not None:
        y = y * np.asarray(scale, dtype=np.float64).reshape(-1, 1)
    return y


def oracle_bwd_bias_scale(x, dy, bias=None, scale=None):
    """Returns (dx [rows, 2n], dbias [2n] or None, dscale [rows] or None)."""
    x = np.asarray(x, dtype=np.float64)
    x2 = x.reshape(-1, x.shape[-1])
    z = x2 + (0.0 if bias is None else np.asarray(bias, dtype=np.float64).reshape(1, -1))
    dy = np.asarray(dy, dtype=np.float64).reshape(z.shape[0], -1)
    s = None if scale is None else np.asarray(scale, dtype=np.float64).reshape(-1, 1)
    dx = oracle_bwd(z, dy if s is None else dy * s)
    dbias = None if bias is None else dx.sum(axis=0)
    dscale = None if scale is None else (dy * oracle_fwd(z)).sum(axis=1)
    return dx, dbias, dscale


# --------------------------------------------------------------------------
# fc1 projection with the SwiGLU as its epilogue
# --------------------------------------------------------------------------
# Liger-Kernel Megatron SwiGLU page, §Background: the packed [tokens, 2n]
# tensor is the output of one fc1 projection (Megatron's ColumnParallelLinear).
# Its weight W is [2n, hidden] in the Linear layout (row j holds output column
# j's weights), so x = A @ W.T, with the gate columns from rows [0, n) of W and
# the up columns from rows [n, 2n). The fused variant computes
#     y = silu(A @ W[:n].T) * (A @ W[n:].T)
# without forming x (the "MLP1 with activation" of the Liger-Kernel test/cute
# page, §MLP1 numerical reference). Products of the inputs are exact in
# float64 for bf16 inputs; the sums are numpy's float64 matmul.

def oracle_fc1(a, w) -> np.ndarray:
    """x = A @ W.T in float64: A [m, k], W [2n, k] -> [m, 2n]."""
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return a @ w.T


def oracle_fc1_swiglu(a, w) -> np.ndarray:
    """y = silu(A @ W[:n].T) * (A @ W[n:].T), float64 [m, n]."""
    return oracle_fwd(oracle_fc1(a, w))


# --------------------------------------------------------------------------
# Comparison targets
# --------------------------------------------------------------------------

def round_f64_to_bf16_bits(v) -> np.ndarray:
    """Correctly rounded bf16 (nearest, ties to even) of float64 values, as
    uint16 bit patterns. One rounding, straight from float64.

    bf16 keeps 8 significant bits. A magnitude a in [2^(e-1), 2^e) therefore
    sits on a grid of spacing 2^(e-8); below the smallest normal 2^-126 the
    grid is the subnormal spacing 2^-133. Scaling a onto that grid is a power
    of two (exact), numpy's rint rounds to the nearest integer with ties to
    even (exact, the scaled value is below 2^9), and scaling back is exact.
    A result of 2^128 or more is an overflow to infinity. NaN maps to the
    quiet NaN 0x7FC0 with the input's sign.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    finite = np.isfinite(a)
    af = np.where(finite, a, 0.0)
    _, e = np.frexp(af)                       # af = m * 2^e, m in [0.5, 1)
    qexp = np.maximum(e.astype(np.int64) - 8, -133)
    k = np.ldexp(af, -qexp)                   # exact
    r = np.rint(k)                            # nearest, ties to even
    val = np.ldexp(r, qexp)                   # exact, a bf16 value or >= 2^128
    with np.errstate(over="ignore"):
        f32 = val.astype(np.float32)          # exact below 2^128, inf at 2^128
    mag = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    mag = np.where(np.isinf(a), np.uint16(0x7F80), mag)
    mag = np.where(np.isnan(a), np.uint16(0x7FC0), mag)
    sign = np.where(np.signbit(v), np.uint16(0x8000), np.uint16(0))
    return (mag | sign).astype(np.uint16)


def bf16_ordinal(bits) -> np.ndarray:
    """Map bf16 patterns onto a monotone integer line: consecutive bf16
    values differ by 1, and +0 and -0 both map to 0."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_distance(a_bits, b_bits) -> np.ndarray:
    """Number of bf16 steps between two finite patterns (0 for +0 vs -0)."""
    return np.abs(bf16_ordinal(a_bits) - bf16_ordinal(b_bits))
