"""Two-tensor SwiGLU on padded views (needs an MI355X).

The two-tensor forward and backward (Liger-Kernel Megatron SwiGLU page,
§Background: the existing op takes gate and up as separate tensors) accept
any row stride >= n. Here every operand -- gate, up, dy and the outputs y,
dgate, dup -- is the first n columns of a wider buffer whose base and row
stride are 16-byte aligned, so the pointers and strides alone would allow
16-byte accesses while n is not a multiple of 16 bytes. Every element is
compared with the oracle, the in-place backward must give the out-of-place
bits, and the padding columns (NaN canaries) must be left untouched.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import swiglu_activation_amd as sw
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

ROWS = 41


def _say(*a):
    print(*a, flush=True)


def _padded_width(n: int, esz: int) -> int:
    """Row width of the backing buffer: n plus at least one canary column,
    rounded up to 16 bytes."""
    per = 16 // esz
    return -(-(n + 1) // per) * per


def _draw(rows, n, dtype, seed):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((rows, n)) * 3.0
    u = rng.standard_normal((rows, n))
    d = rng.standard_normal((rows, n))
    if dtype == "fp32":
        return g.astype(np.float32), u.astype(np.float32), d.astype(np.float32)
    return (oracle.round_f64_to_bf16_bits(g), oracle.round_f64_to_bf16_bits(u),
            oracle.round_f64_to_bf16_bits(d))


def _padded(host, dtype, n, width):
    """A [rows, width] NaN-filled buffer with host copied into its first n
    columns; returns (buffer, view)."""
    rows = host.shape[0]
    buf = torch.full((rows, width), float("nan"), dtype=gu.torch_dtype(dtype), device="cuda")
    view = buf[:, :n]
    if host is not None:
        view.copy_(gu.to_dev(host, dtype))
    return buf, view


def _empty_padded(rows, dtype, n, width):
    buf = torch.full((rows, width), float("nan"), dtype=gu.torch_dtype(dtype), device="cuda")
    return buf, buf[:, :n]


def _canaries_intact(buf, n):
    return bool(torch.isnan(buf[:, n:].float()).all())


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n", [1, 3, 5, 7, 9, 12, 127, 1001, 4100])
def test_two_tensor_padded_views(n, dtype):
    esz = 4 if dtype == "fp32" else 2
    width = _padded_width(n, esz)
    _say(f"[two-tensor padded] n={n} {dtype} rows={ROWS} width={width}")
    g_h, u_h, d_h = _draw(ROWS, n, dtype, seed=1000 + n)
    gb, g = _padded(g_h, dtype, n, width)
    ub, u = _padded(u_h, dtype, n, width)
    db, dy = _padded(d_h, dtype, n, width)
    assert g.data_ptr() % 16 == 0 and g.stride(0) * esz % 16 == 0

    yb, y = _empty_padded(ROWS, dtype, n, width)
    dgb, dg = _empty_padded(ROWS, dtype, n, width)
    dub, du = _empty_padded(ROWS, dtype, n, width)
    sw.swiglu_silu_mul_fwd(g, u, y)
    sw.swiglu_silu_mul_bwd(dy, g, u, dg, du)
    # in place on copies of the padded inputs
    gib, gi = _padded(g_h, dtype, n, width)
    uib, ui = _padded(u_h, dtype, n, width)
    sw.swiglu_silu_mul_bwd(dy, gi, ui, in_place=True)
    torch.cuda.synchronize()

    for buf, what in ((yb, "y"), (dgb, "dgate"), (dub, "dup"), (gib, "gate in place"),
                      (uib, "up in place"), (gb, "gate"), (ub, "up"), (db, "dy")):
        assert _canaries_intact(buf, n), f"padding of {what} was written"
    assert gu.bits_equal(gi, dg) and gu.bits_equal(ui, du), "in-place differs from out of place"
    assert np.array_equal(gu.from_dev(g), g_h) and np.array_equal(gu.from_dev(u), u_h), \
        "out-of-place backward touched its inputs"

    xf = np.concatenate([oracle.widen(g_h, dtype), oracle.widen(u_h, dtype)], 1)
    dyf = oracle.widen(d_h, dtype)
    dref = oracle.oracle_bwd(xf, dyf)
    st = {"fwd": gu.compare(gu.from_dev(y), oracle.oracle_fwd(xf), dtype, "y"),
          "dgate": gu.compare(gu.from_dev(dg), dref[:, :n], dtype, "dgate"),
          "dup": gu.compare(gu.from_dev(du), dref[:, n:], dtype, "dup")}
    msgs = [str(s) for s in st.values()]
    _say("   " + "\n   ".join(msgs))
    assert all(s.ok() for s in st.values()), "\n".join(msgs)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_two_tensor_mixed_padding(dtype):
    """Each operand padded differently (and one of them packed), n = 13:
    the access width must suit every operand and n at once."""
    esz = 4 if dtype == "fp32" else 2
    n = 13
    _say(f"[two-tensor mixed padding] {dtype}")
    g_h, u_h, d_h = _draw(ROWS, n, dtype, seed=77)
    gb, g = _padded(g_h, dtype, n, _padded_width(n, esz))
    ub, u = _padded(u_h, dtype, n, 40)
    dy = gu.to_dev(d_h, dtype)                              # packed, stride n
    yb, y = _empty_padded(ROWS, dtype, n, 24)
    dgb, dg = _empty_padded(ROWS, dtype, n, 16)
    dub, du = _empty_padded(ROWS, dtype, n, 32)
    sw.swiglu_silu_mul_fwd(g, u, y)
    sw.swiglu_silu_mul_bwd(dy, g, u, dg, du)
    torch.cuda.synchronize()
    for buf in (yb, dgb, dub, gb, ub):
        assert _canaries_intact(buf, n)
    xf = np.concatenate([oracle.widen(g_h, dtype), oracle.widen(u_h, dtype)], 1)
    dref = oracle.oracle_bwd(xf, oracle.widen(d_h, dtype))
    st = [gu.compare(gu.from_dev(y), oracle.oracle_fwd(xf), dtype, "y"),
          gu.compare(gu.from_dev(dg), dref[:, :n], dtype, "dgate"),
          gu.compare(gu.from_dev(du), dref[:, n:], dtype, "dup")]
    _say("   " + "\n   ".join(str(s) for s in st))
    assert all(s.ok() for s in st)
