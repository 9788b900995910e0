"""Bias and per-token scale variants vs the oracle (needs an MI355X).

Bars: y and dx elementwise as for the base op (fp32 1e-5 relative, bf16
2 ulp). dbias and dscale are fp32 sums accumulated in fp32 in a fixed order;
their bar is |got - ref| <= 1e-5 * sum |terms| (the float64 sum of the terms'
magnitudes), which bounds fp32 accumulation of up to millions of terms with
a wide margin and stays meaningful when the sum cancels.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
import swiglu_activation_amd as sw
from swiglu_activation_amd.autograd import MegatronSwiGLU, weighted_swiglu
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
SUM_TOL = 1e-5


def _to_store(v, dtype):
    return v.astype(np.float32) if dtype == "fp32" else oracle.round_f64_to_bf16_bits(v)


def _make(rows, n, dtype, seed, bias=True, scale=True, x_h=None, dy_h=None):
    rng = np.random.default_rng(seed)
    if x_h is None:
        g, u = rng.standard_normal((2, rows, n))
        x_h = _to_store(np.concatenate([g * 3, u], 1), dtype)
        dy_h = _to_store(rng.standard_normal((rows, n)), dtype)
    b_h = _to_store(rng.standard_normal(2 * n) * 0.5, dtype) if bias else None
    s_h = rng.uniform(0.05, 1.0, rows).astype(np.float32) if scale else None
    return x_h, dy_h, b_h, s_h


def _refs(x_h, dy_h, b_h, s_h, dtype):
    xf, dyf = oracle.widen(x_h, dtype), oracle.widen(dy_h, dtype)
    bf = None if b_h is None else oracle.widen(b_h, dtype)
    sf = None if s_h is None else s_h.astype(np.float64)
    y = oracle.oracle_fwd_bias_scale(xf, bf, sf)
    dx, db, ds = oracle.oracle_bwd_bias_scale(xf, dyf, bf, sf)
    # magnitudes of the summed terms, for the bars of dbias and dscale
    z = xf + (0 if bf is None else bf)
    n = z.shape[1] // 2
    db_abs = np.abs(dx).sum(axis=0) if bf is not None else None
    ds_abs = np.abs(dyf * oracle.oracle_fwd(z)).sum(axis=1) if sf is not None else None
    return y, dx, db, ds, db_abs, ds_abs


def _check_sum(got, ref, absref, what):
    got = got.detach().cpu().numpy().astype(np.float64).reshape(ref.shape)
    err = np.abs(got - ref)
    bound = SUM_TOL * absref + 1e-30
    worst = float(np.max(err / bound))
    print(f"    {what}: {ref.size} sums, worst {worst:.3g} of the bar", flush=True)
    assert np.all(err <= bound), (what, worst)


def _check_elem(got, ref, dtype, what):
    st = gu.compare(gu.from_dev(got).reshape(ref.shape), ref, dtype, what)
    print("   ", st, flush=True)
    assert st.ok(), str(st)


def _run_and_check(x_h, dy_h, b_h, s_h, dtype, in_place=False, shape=None):
    rows, n = x_h.shape[0], x_h.shape[1] // 2
    y_ref, dx_ref, db_ref, ds_ref, db_abs, ds_abs = _refs(x_h, dy_h, b_h, s_h, dtype)
    x = gu.to_dev(x_h, dtype)
    dy = gu.to_dev(dy_h, dtype)
    if shape is not None:
        x, dy = x.reshape(shape), dy.reshape(shape[:-1] + (n,))
    b = None if b_h is None else gu.to_dev(b_h, dtype)
    s = None if s_h is None else torch.from_numpy(s_h).cuda().reshape(x.shape[:-1])
    y = sw.swiglu_gateup_bias_scale_fwd(x, b, s)
    xin = x.clone() if in_place else x
    dx, db, ds = sw.swiglu_gateup_bias_scale_bwd(dy, xin, b, s, in_place=in_place)
    torch.cuda.synchronize()
    _check_elem(y, y_ref, dtype, "fwd")
    _check_elem(dx, dx_ref, dtype, "dx")
    if b_h is not None:
        _check_sum(db, db_ref, db_abs, "dbias")
    if s_h is not None:
        _check_sum(ds, ds_ref, ds_abs, "dscale")
    return y, dx, db, ds


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("variant", ["bias", "scale", "both", "neither"])
@pytest.mark.parametrize("in_place", [False, True])
def test_bias_scale_parity(dtype, variant, in_place):
    """Ragged everything: 777 rows (not a multiple of the row group or the
    unroll), n = 1100 (a partial last column tile, 8-byte bf16 accesses)."""
    print(f"[bias/scale] {dtype} {variant} in_place={in_place}", flush=True)
    bias = variant in ("bias", "both")
    scale = variant in ("scale", "both")
    x_h, dy_h, b_h, s_h = _make(777, 1100, dtype, seed=41, bias=bias, scale=scale)
    _run_and_check(x_h, dy_h, b_h, s_h, dtype, in_place=in_place)


def test_in_place_and_repeat_are_bitwise_identical():
    x_h, dy_h, b_h, s_h = _make(515, 2048, "bf16", seed=42)
    x, dy = gu.to_dev(x_h, "bf16"), gu.to_dev(dy_h, "bf16")
    b, s = gu.to_dev(b_h, "bf16"), torch.from_numpy(s_h).cuda()
    r1 = sw.swiglu_gateup_bias_scale_bwd(dy, x, b, s)
    r2 = sw.swiglu_gateup_bias_scale_bwd(dy, x, b, s)
    xc = x.clone()
    r3 = sw.swiglu_gateup_bias_scale_bwd(dy, xc, b, s, in_place=True)
    torch.cuda.synchronize()
    for a, c in ((r1, r2), (r1, r3)):
        assert gu.bits_equal(a[0], c[0])
        assert torch.equal(a[1].view(torch.int32), c[1].view(torch.int32))
        assert torch.equal(a[2].view(torch.int32), c[2].view(torch.int32))


def test_neither_matches_base_op():
    x_h, dy_h, _, _ = _make(300, 4096, "bf16", seed=43, bias=False, scale=False)
    x, dy = gu.to_dev(x_h, "bf16"), gu.to_dev(dy_h, "bf16")
    y1 = sw.swiglu_gateup_bias_scale_fwd(x)
    dx1, _, _ = sw.swiglu_gateup_bias_scale_bwd(dy, x)
    torch.cuda.synchronize()
    assert torch.equal(y1, sw.swiglu_gateup_fwd(x))       # values; zeros may differ in sign
    assert torch.equal(dx1, sw.swiglu_gateup_bwd(dy, x))


def test_fp32_biased_gate_at_the_silu_minimiser():
    """z = x + bias lands within +-2e-3 of g0 = -1 - W(1/e) where the bracket
    1 + z(1 - sigma(z)) has its root: the kernel forms z in fp32 and must
    carry the rounding error of the sum into the root series."""
    print("[bias/scale] fp32 biased root", flush=True)
    rows, n = 64, 4096
    rng = np.random.default_rng(44)
    bias = np.concatenate([rng.standard_normal(n) * 3, rng.standard_normal(n)]).astype(np.float32)
    target = oracle.G0 + rng.uniform(-2e-3, 2e-3, (rows, n))
    g = (target - bias[:n].astype(np.float64)).astype(np.float32)
    u = rng.standard_normal((rows, n)).astype(np.float32)
    x_h = np.concatenate([g, u], 1)
    dy_h = rng.standard_normal((rows, n)).astype(np.float32)
    _run_and_check(x_h, dy_h, bias, None, "fp32")


def test_empty_problems_zero_the_sums():
    b = torch.randn(64, device="cuda").bfloat16()
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    dy = torch.empty(0, 32, dtype=torch.bfloat16, device="cuda")
    _, db, _ = sw.swiglu_gateup_bias_scale_bwd(dy, x, b)
    s = torch.rand(5, device="cuda")
    x0 = torch.empty(5, 0, dtype=torch.bfloat16, device="cuda")
    dy0 = torch.empty(5, 0, dtype=torch.bfloat16, device="cuda")
    _, _, ds = sw.swiglu_gateup_bias_scale_bwd(dy0, x0, None, s)
    torch.cuda.synchronize()
    assert db.shape == (64,) and torch.all(db == 0)
    assert ds.shape == (5,) and torch.all(ds == 0)


def test_argument_errors():
    x = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    dy = torch.zeros(8, 32, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        sw.swiglu_gateup_bias_scale_fwd(x, torch.zeros(63, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        sw.swiglu_gateup_bias_scale_fwd(x, None, torch.zeros(8, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        sw.swiglu_gateup_bias_scale_bwd(dy, x, torch.zeros(64, dtype=torch.bfloat16, device="cuda"),
                                        workspace=torch.zeros(8, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        sw.swiglu_gateup_bias_scale_bwd(dy, x, None, None, want_dbias=True)


def test_autograd_weighted_and_biased():
    x_h, dy_h, b_h, s_h = _make(96, 512, "fp32", seed=45)
    x = gu.to_dev(x_h, "fp32").requires_grad_(True)
    b = gu.to_dev(b_h, "fp32").requires_grad_(True)
    s = torch.from_numpy(s_h).cuda().reshape(96, 1).requires_grad_(True)
    dy = gu.to_dev(dy_h, "fp32")
    weighted_swiglu(x, s, b).backward(dy)
    dx, db, ds = sw.swiglu_gateup_bias_scale_bwd(dy, x.detach(), b.detach(), s.detach())
    torch.cuda.synchronize()
    assert torch.equal(x.grad, dx) and torch.equal(b.grad, db) and torch.equal(s.grad, ds)
    # the module with a bias: bias gradient in the bias dtype
    xb = gu.to_dev(_to_store(np.random.default_rng(1).standard_normal((2, 5, 64)), "bf16"),
                   "bf16").requires_grad_(True)
    bb = torch.randn(64, device="cuda").bfloat16().requires_grad_(True)
    MegatronSwiGLU()(xb, bb).sum().backward()
    torch.cuda.synchronize()
    assert bb.grad.dtype == torch.bfloat16 and xb.grad.shape == xb.shape


@pytest.mark.parametrize("name", ["dense_bf16_s2048_b4_n4096", "inplace_tp_bf16_t8192_n1792",
                                  "odd_fp32_s4096_b1_n11008"])
def test_full_size_workloads_with_bias_and_scale(name):
    """The workloads' own inputs plus a bias ~ N(0, 0.25) and router-like
    scales ~ U(0.05, 1), every output element compared."""
    w = synth.WORKLOADS[name]
    print(f"[bias/scale full] {name}", flush=True)
    x_h, dy_h = synth.make_x(w), synth.make_dy(w)
    _, _, b_h, s_h = _make(w.rows, w.n, w.dtype, seed=46, x_h=x_h, dy_h=dy_h)
    _run_and_check(x_h, dy_h, b_h, s_h, w.dtype, in_place=w.in_place, shape=w.shape)


@pytest.mark.parametrize("dtype,n", [("bf16", 2048), ("fp32", 1024)])
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("in_place", [False, True])
def test_one_shot_backward_matches_row_loop(dtype, n, bias, in_place):
    """Without dbias, wide rows of 16-byte vectors take a one-shot kernel;
    with dbias, the tile kernel (one-shot too, with the column sums added
    across waves in LDS). dx and dscale must be the same bits."""
    print(f"[bias/scale one-shot] {dtype} n={n} bias={bias} in_place={in_place}", flush=True)
    x_h, dy_h, b_h, s_h = _make(515, n, dtype, seed=47, bias=bias, scale=True)
    x, dy = gu.to_dev(x_h, dtype), gu.to_dev(dy_h, dtype)
    b = gu.to_dev(b_h, dtype) if bias else None
    s = torch.from_numpy(s_h).cuda()
    ref_b = gu.to_dev(b_h, dtype) if bias else gu.to_dev(np.zeros(2 * n, x_h.dtype), dtype)
    # row loop (dbias requested; a zero bias when the case has none)
    dx_l, _, ds_l = sw.swiglu_gateup_bias_scale_bwd(dy, x.clone(), ref_b, s, want_dbias=True,
                                                    in_place=in_place)
    # one shot
    dx_o, db_o, ds_o = sw.swiglu_gateup_bias_scale_bwd(dy, x.clone(), b, s, want_dbias=False,
                                                       in_place=in_place)
    torch.cuda.synchronize()
    assert db_o is None
    assert gu.bits_equal(dx_l, dx_o)
    assert torch.equal(ds_l.view(torch.int32), ds_o.view(torch.int32))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_scale_only_wide_rows_parity(dtype):
    """The per-token-scale form without a bias (routed experts) on wide rows:
    the one-shot backward against the oracle."""
    print(f"[bias/scale scale only] {dtype}", flush=True)
    x_h, dy_h, b_h, s_h = _make(300, 4096, dtype, seed=48, bias=False, scale=True)
    _run_and_check(x_h, dy_h, b_h, s_h, dtype)
    _run_and_check(x_h, dy_h, b_h, s_h, dtype, in_place=True)


@pytest.mark.parametrize("dtype,rows,n", [("bf16", 777, 1096), ("fp32", 777, 260),
                                          ("bf16", 64, 512), ("fp32", 129, 4100)])
@pytest.mark.parametrize("scale", [False, True])
@pytest.mark.parametrize("in_place", [False, True])
def test_tile_backward_ragged(dtype, rows, n, scale, in_place):
    """The dbias backward on 16-byte rows (tile kernel: 64-vector chunks of
    64-row groups) with a partial last chunk (nv = 137, 65, 1025) and a
    partial last row group, against the oracle; one exact chunk and group
    (bf16 64 x 512)."""
    print(f"[bias/scale tile] {dtype} rows={rows} n={n} scale={scale} in_place={in_place}",
          flush=True)
    x_h, dy_h, b_h, s_h = _make(rows, n, dtype, seed=49, bias=True, scale=scale)
    _run_and_check(x_h, dy_h, b_h, s_h, dtype, in_place=in_place)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_tile_and_row_loop_give_the_same_dx(dtype):
    """The same problem through the tile kernel (16-byte aligned rows) and
    through the row-loop kernel (the rows moved by one element, so only
    narrower accesses fit): dx is computed per element by the same function,
    so it is the same bits; dbias and dscale are summed in other orders and
    each meets the oracle's bar."""
    rows, n = 300, 2048
    x_h, dy_h, b_h, s_h = _make(rows, n, dtype, seed=50)
    y_ref, dx_ref, db_ref, ds_ref, db_abs, ds_abs = _refs(x_h, dy_h, b_h, s_h, dtype)
    x, dy = gu.to_dev(x_h, dtype), gu.to_dev(dy_h, dtype)
    b, s = gu.to_dev(b_h, dtype), torch.from_numpy(s_h).cuda()
    # misaligned copies: one element into a wider buffer, row stride 2n + 1
    xm_buf = torch.empty(rows, 2 * n + 1, dtype=x.dtype, device="cuda")
    xm = xm_buf[:, 1:]
    xm.copy_(x)
    dxm_buf = torch.empty(rows, 2 * n + 1, dtype=x.dtype, device="cuda")
    dxm = dxm_buf[:, 1:]
    dx_t, db_t, ds_t = sw.swiglu_gateup_bias_scale_bwd(dy, x, b, s)
    dx_l, db_l, ds_l = sw.swiglu_gateup_bias_scale_bwd(dy, xm, b, s, dx=dxm)
    torch.cuda.synchronize()
    assert gu.bits_equal(dx_t, dx_l.contiguous())
    _check_elem(dx_t, dx_ref, dtype, "dx (tile)")
    for db, ds, what in ((db_t, ds_t, "tile"), (db_l, ds_l, "row loop")):
        _check_sum(db, db_ref, db_abs, f"dbias ({what})")
        _check_sum(ds, ds_ref, ds_abs, f"dscale ({what})")


@pytest.mark.parametrize("in_place", [False, True])
def test_fp32_gates_below_the_normal_range_of_sigma(in_place):
    """fp32, biased gates z in [-100, -84]: sigma(z) ~ e^z is an fp32 subnormal
    below z ~ -87.3 while silu(z) u stays normal down to z ~ -91.8. Every
    output whose reference is a normal fp32 number meets the 1e-5 relative
    bar, every subnormal one meets it up to one subnormal step (|got - ref| <=
    1e-5 |ref| + 2^-149: the one rounding into the subnormal range), and
    dbias and dscale meet their bars."""
    print(f"[bias/scale fp32 low gates] in_place={in_place}", flush=True)
    rng = np.random.default_rng(51)
    rows, n = 128, 1024
    bias = rng.uniform(-1.0, 1.0, 2 * n)
    g = rng.uniform(-100.0, -84.0, (rows, n)) - bias[:n]
    u = rng.choice([-1.0, 1.0], (rows, n)) * rng.uniform(1.0, 2.0, (rows, n))
    dy = rng.choice([-1.0, 1.0], (rows, n)) * rng.uniform(1.0, 2.0, (rows, n))
    x_h = np.concatenate([g, u], 1).astype(np.float32)
    dy_h = dy.astype(np.float32)
    b_h = bias.astype(np.float32)
    s_h = rng.uniform(0.5, 1.0, rows).astype(np.float32)
    y_ref, dx_ref, db_ref, ds_ref, db_abs, ds_abs = _refs(x_h, dy_h, b_h, s_h, "fp32")
    x, dyt = gu.to_dev(x_h, "fp32"), gu.to_dev(dy_h, "fp32")
    b, s = gu.to_dev(b_h, "fp32"), torch.from_numpy(s_h).cuda()
    y = sw.swiglu_gateup_bias_scale_fwd(x, b, s)
    dx, db, ds = sw.swiglu_gateup_bias_scale_bwd(dyt, x.clone() if in_place else x, b, s,
                                                 in_place=in_place)
    torch.cuda.synchronize()
    tiny = 2.0 ** -126
    counts = {}
    for got_t, ref, what in ((y, y_ref, "fwd"), (dx, dx_ref, "dx")):
        got = gu.from_dev(got_t).reshape(ref.shape).astype(np.float64)
        normal = np.abs(ref) >= tiny
        rel = np.abs(got - ref)[normal] / np.abs(ref[normal])
        sub = ~normal & (ref != 0)
        over = (np.abs(got - ref)[sub] - 1e-5 * np.abs(ref[sub])) / 2.0 ** -149
        counts[what] = (int(normal.sum()), int(sub.sum()))
        print(f"    {what}: {normal.sum()} normal (max rel {rel.max():.3g}), {sub.sum()} subnormal "
              f"(max excess over 1e-5 |ref|: {over.max() if over.size else 0:.3g} steps)", flush=True)
        assert rel.max() <= 1e-5 and (over.size == 0 or over.max() <= 1.0), what
        assert np.all(got[ref == 0] == 0)
    assert counts["fwd"][0] > 0 and counts["fwd"][1] > 0
    _check_sum(db, db_ref, db_abs, "dbias")
    _check_sum(ds, ds_ref, ds_abs, "dscale")
