"""HIP path vs the CPU oracle, element by element (needs an MI355X).

Every workload runs at its full size in the same launch configuration the
bench uses, and every output element is compared with the oracle: forward,
out-of-place backward and in-place backward. Smaller cases cover the ragged
tail of the grid walk, odd widths (narrow accesses), strided and misaligned
views, 3D inputs, empty problems and 64-bit offsets.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
import swiglu_activation_amd as sw
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _inputs(w: synth.Workload, rows=None):
    r1 = w.rows if rows is None else rows
    x_h = synth.make_x(w, 0, r1)
    dy_h = synth.make_dy(w, 0, r1)
    return x_h, dy_h


def _run_all(x, dy):
    """fwd, out-of-place bwd, in-place bwd (on a clone); returns device tensors."""
    y = sw.swiglu_gateup_fwd(x)
    dx = sw.swiglu_gateup_bwd(dy, x)
    x_ip = x.clone()
    dx_ip = sw.swiglu_gateup_bwd(dy, x_ip, in_place=True)
    torch.cuda.synchronize()
    assert dx_ip.data_ptr() == x_ip.data_ptr()
    return y, dx, dx_ip


def _assert_stats(stats):
    msgs = [str(s) for s in stats.values()]
    _say("   " + "\n   ".join(msgs))
    assert all(s.ok() for s in stats.values()), "\n".join(msgs)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_full_parity(name):
    """All of fwd / bwd / bwd in_place on every element of a full-size workload."""
    w = synth.WORKLOADS[name]
    _say(f"[parity] {name}: x {w.shape} {w.dtype}, n={w.n}")
    x_h, dy_h = _inputs(w)
    x = gu.to_dev(x_h, w.dtype).reshape(w.shape)
    dy = gu.to_dev(dy_h, w.dtype).reshape(w.shape[:-1] + (w.n,))
    y, dx, dx_ip = _run_all(x, dy)
    assert gu.bits_equal(dx, dx_ip), "in-place backward differs from out-of-place"
    assert np.array_equal(gu.from_dev(x).reshape(x_h.shape), x_h), "out-of-place bwd touched x"
    outs = {"fwd": ("fwd", gu.from_dev(y).reshape(w.rows, w.n)),
            "bwd": ("bwd", gu.from_dev(dx).reshape(w.rows, 2 * w.n))}
    del y, dx, dx_ip
    _assert_stats(gu.compare_workload_chunks(w, x_h, dy_h, outs))


def test_repeat_runs_are_bitwise_identical():
    w = synth.WORKLOADS["dense_bf16_s2048_b4_n4096"]
    x_h, dy_h = _inputs(w, 1024)
    x = gu.to_dev(x_h, w.dtype)
    dy = gu.to_dev(dy_h, w.dtype)
    a = _run_all(x, dy)
    b = _run_all(x, dy)
    for p, q in zip(a, b):
        assert gu.bits_equal(p, q)


def _random_case(rows, n, dtype, seed, gate_scale=3.0):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((rows, n)) * gate_scale
    u = rng.standard_normal((rows, n))
    d = rng.standard_normal((rows, n))
    if dtype == "fp32":
        x_h = np.concatenate([g, u], 1).astype(np.float32)
        dy_h = d.astype(np.float32)
    else:
        x_h = oracle.round_f64_to_bf16_bits(np.concatenate([g, u], 1))
        dy_h = oracle.round_f64_to_bf16_bits(d)
    return x_h, dy_h


def _check_case(x_h, dy_h, dtype, x=None, dy=None, what=""):
    rows, n = x_h.shape[0], x_h.shape[1] // 2
    x = gu.to_dev(x_h, dtype) if x is None else x
    dy = gu.to_dev(dy_h, dtype) if dy is None else dy
    y, dx, dx_ip = _run_all(x, dy)
    assert gu.bits_equal(dx, dx_ip)
    xf, dyf = oracle.widen(x_h, dtype), oracle.widen(dy_h, dtype)
    st = {"fwd": gu.compare(gu.from_dev(y).reshape(rows, n), oracle.oracle_fwd(xf), dtype, what + " fwd"),
          "bwd": gu.compare(gu.from_dev(dx).reshape(rows, 2 * n), oracle.oracle_bwd(xf, dyf), dtype,
                            what + " bwd")}
    _assert_stats(st)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n", [1, 2, 3, 7, 8, 127, 129, 1001, 4100])
def test_odd_and_small_widths(n, dtype):
    """Widths that force 8-, 4- and 2-byte or single-element accesses."""
    rows = 37
    _say(f"[odd] n={n} {dtype}")
    x_h, dy_h = _random_case(rows, n, dtype, seed=n)
    _check_case(x_h, dy_h, dtype, what=f"n={n}")


@pytest.mark.parametrize("rows", [1, 3, 1023, 1025, 4097])
def test_ragged_grid_tails(rows):
    """Row counts around the grid span's boundaries, several grid passes."""
    n = 1792
    _say(f"[tail] rows={rows}")
    x_h, dy_h = _random_case(rows, n, "bf16", seed=rows)
    _check_case(x_h, dy_h, "bf16", what=f"rows={rows}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_strided_views_and_guard_columns(dtype):
    """Row strides above the width: results equal the contiguous ones and the
    columns between rows are never written."""
    rows, n, pad = 300, 520, 24
    _say(f"[strided] {dtype}")
    tdt = gu.torch_dtype(dtype)
    x_h, dy_h = _random_case(rows, n, dtype, seed=5)
    x_c, dy_c = gu.to_dev(x_h, dtype), gu.to_dev(dy_h, dtype)
    y_c = sw.swiglu_gateup_fwd(x_c)
    dx_c = sw.swiglu_gateup_bwd(dy_c, x_c)

    canary = torch.full((), float("nan"), dtype=tdt, device="cuda")
    xb = torch.empty(rows, 2 * n + pad, dtype=tdt, device="cuda").fill_(canary)
    x = xb[:, :2 * n]
    x.copy_(x_c)
    dyb = torch.empty(rows, n + pad, dtype=tdt, device="cuda").fill_(canary)
    dy = dyb[:, pad:]
    dy.copy_(dy_c)
    yb = torch.empty(rows, n + pad, dtype=tdt, device="cuda").fill_(canary)
    y = yb[:, pad // 2: pad // 2 + n]
    dxb = torch.empty(rows, 2 * n + pad, dtype=tdt, device="cuda").fill_(canary)
    dx = dxb[:, pad:]
    sw.swiglu_gateup_fwd(x, y)
    sw.swiglu_gateup_bwd(dy, x, dx)
    sw.swiglu_gateup_bwd(dy, x, in_place=True)
    torch.cuda.synchronize()
    assert gu.bits_equal(y, y_c) and gu.bits_equal(dx, dx_c) and gu.bits_equal(x, dx_c)
    assert torch.isnan(yb[:, :pad // 2]).all() and torch.isnan(yb[:, pad // 2 + n:]).all()
    assert torch.isnan(dxb[:, :pad]).all()
    assert torch.isnan(xb[:, 2 * n:]).all()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("offset", [1, 2, 3])
def test_misaligned_base_pointers(dtype, offset):
    rows, n = 65, 256
    _say(f"[misaligned] {dtype} +{offset}")
    tdt = gu.torch_dtype(dtype)
    x_h, dy_h = _random_case(rows, n, dtype, seed=offset)
    xb = torch.empty(rows * 2 * n + offset, dtype=tdt, device="cuda")
    x = xb[offset:].view(rows, 2 * n)
    x.copy_(gu.to_dev(x_h, dtype))
    dyb = torch.empty(rows * n + 2 * offset, dtype=tdt, device="cuda")
    dy = dyb[2 * offset:].view(rows, n)
    dy.copy_(gu.to_dev(dy_h, dtype))
    _check_case(x_h, dy_h, dtype, x=x, dy=dy, what=f"+{offset}")


def test_three_d_and_empty_inputs():
    x_h, dy_h = _random_case(4 * 6, 64, "bf16", seed=1)
    x = gu.to_dev(x_h, "bf16").reshape(4, 6, 128)
    dy = gu.to_dev(dy_h, "bf16").reshape(4, 6, 64)
    y = sw.swiglu_gateup_fwd(x)
    assert y.shape == (4, 6, 64)
    dx = sw.swiglu_gateup_bwd(dy, x)
    assert dx.shape == (4, 6, 128)
    y2 = sw.swiglu_gateup_fwd(x.reshape(24, 128))
    assert gu.bits_equal(y.reshape(24, 64), y2)
    for shape in [(0, 128), (5, 0), (0, 3, 16)]:
        e = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        ye = sw.swiglu_gateup_fwd(e)
        assert ye.shape == shape[:-1] + (shape[-1] // 2,)
        de = sw.swiglu_gateup_bwd(torch.empty(ye.shape, dtype=torch.bfloat16, device="cuda"), e)
        assert de.shape == e.shape
    torch.cuda.synchronize()


def test_argument_errors_with_real_tensors():
    x = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        sw.swiglu_gateup_fwd(x.half())                     # fp16 is not supported
    with pytest.raises(ValueError):
        sw.swiglu_gateup_fwd(x, x[:, :32])                 # y overlaps x
    with pytest.raises(ValueError):
        sw.swiglu_gateup_bwd(x[:, :32], x, x)              # dx overlaps x
    with pytest.raises(ValueError):
        sw.swiglu_gateup_bwd(x[:, 8:40], x, in_place=True)  # dy overlaps x
    with pytest.raises(ValueError):
        sw.swiglu_gateup_fwd(torch.zeros(8, 63, dtype=torch.bfloat16, device="cuda"))


def test_64bit_row_offsets():
    """Rows more than 2^32 elements apart (byte offsets beyond 8 GiB)."""
    rows, n = 3, 64
    stride = (1 << 32) + 64
    _say("[64-bit] allocating", (rows - 1) * stride + 2 * n, "bf16 elements")
    buf = torch.zeros((rows - 1) * stride + 2 * n, dtype=torch.bfloat16, device="cuda")
    x = torch.as_strided(buf, (rows, 2 * n), (stride, 1))
    x_h, dy_h = _random_case(rows, n, "bf16", seed=64)
    x.copy_(gu.to_dev(x_h, "bf16"))
    dy = gu.to_dev(dy_h, "bf16")
    y = sw.swiglu_gateup_fwd(x)
    dx = sw.swiglu_gateup_bwd(dy, x)
    torch.cuda.synchronize()
    xf, dyf = oracle.widen(x_h, "bf16"), oracle.widen(dy_h, "bf16")
    st = {"fwd": gu.compare(gu.from_dev(y), oracle.oracle_fwd(xf), "bf16", "fwd"),
          "bwd": gu.compare(gu.from_dev(dx), oracle.oracle_bwd(xf, dyf), "bf16", "bwd")}
    sw.swiglu_gateup_bwd(dy, x, in_place=True)
    torch.cuda.synchronize()
    assert gu.bits_equal(x, dx)
    del buf, x
    _assert_stats(st)


def test_runs_on_the_callers_stream():
    x_h, dy_h = _random_case(512, 2048, "bf16", seed=3)
    x, dy = gu.to_dev(x_h, "bf16"), gu.to_dev(dy_h, "bf16")
    ref_y = sw.swiglu_gateup_fwd(x)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = sw.swiglu_gateup_fwd(x)
    s.synchronize()
    assert gu.bits_equal(y, ref_y)
    y2 = torch.empty_like(ref_y)
    sw.swiglu_gateup_fwd(x, y2, stream=s)
    s.synchronize()
    assert gu.bits_equal(y2, ref_y)


@pytest.mark.parametrize("rows,n", [(65535 + 100, 2048), (800_003, 200)])
def test_launch_chunks_and_large_flat_index(rows, n):
    """Wide rows past 65535 (the forward and backward split into two
    launches), and narrow rows whose flat lane index passes 2^24 (an fp32
    quotient would no longer be exact there). Inputs are drawn on the device
    (seeded torch generator, rounded to bf16); rows around the launch
    boundary, the last rows and a random sample are compared with the
    oracle; the in-place backward must equal the out-of-place one bitwise."""
    _say(f"[chunks] rows={rows} n={n}")
    gen = torch.Generator(device="cuda").manual_seed(rows + n)
    x = (torch.randn(rows, 2 * n, device="cuda", generator=gen) * 2).bfloat16()
    dy = torch.randn(rows, n, device="cuda", generator=gen).bfloat16()
    y = sw.swiglu_gateup_fwd(x)
    dx = sw.swiglu_gateup_bwd(dy, x)
    xi = x.clone()
    sw.swiglu_gateup_bwd(dy, xi, in_place=True)
    torch.cuda.synchronize()
    assert gu.bits_equal(xi, dx)
    rng = np.random.default_rng(rows)
    pick = np.unique(np.concatenate([np.arange(0, 4), np.arange(65530, 65541),
                                     np.arange(rows - 4, rows), rng.choice(rows, 64, replace=False)]))
    pick = pick[pick < rows]
    idx = torch.from_numpy(pick).cuda()
    x_h, dy_h = gu.from_dev(x[idx]), gu.from_dev(dy[idx])
    xf, dyf = oracle.widen(x_h, "bf16"), oracle.widen(dy_h, "bf16")
    st = {"fwd": gu.compare(gu.from_dev(y[idx]), oracle.oracle_fwd(xf), "bf16", "fwd"),
          "bwd": gu.compare(gu.from_dev(dx[idx]), oracle.oracle_bwd(xf, dyf), "bf16", "bwd")}
    del x, dy, y, dx, xi
    _assert_stats(st)
