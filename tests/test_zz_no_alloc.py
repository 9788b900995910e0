"""The allocation-free bias/scale backward (needs an MI355X).

swiglu_gateup_bias_scale_bwd_noalloc is called through the C ABI (ctypes,
raw device pointers) and compared bit for bit with
swiglu_gateup_bias_scale_bwd given a workspace of its own: dx, dbias and
dscale. Two calls in a row, the second smaller than the first (the static
scratch then still holds the first call's partials), then an in-place call,
and a problem past the scratch limit, which must be refused before anything
runs.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import swiglu_activation_amd as sw
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _inputs(rows, n, dtype, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    tdt = gu.torch_dtype(dtype)
    x = (torch.randn(rows, 2 * n, device="cuda", generator=gen) * 2).to(tdt)
    dy = torch.randn(rows, n, device="cuda", generator=gen).to(tdt)
    bias = (torch.randn(2 * n, device="cuda", generator=gen) * 0.5).to(tdt)
    scale = torch.rand(rows, device="cuda", generator=gen) + 0.25
    return x, dy, bias, scale


def _dt(dtype):
    return sw.SWIGLU_DTYPE_F32 if dtype == "fp32" else sw.SWIGLU_DTYPE_BF16


def _with_workspace(lib, x, dy, bias, scale, want_db, want_ds, in_place, dtype):
    rows, n = x.shape[0], x.shape[1] // 2
    dx = None if in_place else torch.empty_like(x)
    dbias = torch.empty(2 * n, dtype=torch.float32, device="cuda") if want_db else None
    dscale = torch.empty(rows, dtype=torch.float32, device="cuda") if want_ds else None
    need = lib.swiglu_gateup_bias_scale_workspace_size(rows, n, int(want_db), int(want_ds))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    st = lib.swiglu_gateup_bias_scale_bwd(
        _p(dy), n, _p(x), 2 * n, _p(bias), _p(scale), 1, _p(dx), 2 * n, _p(dbias), _p(dscale), 1,
        _p(ws), need, rows, n, _dt(dtype), int(in_place), _stream())
    assert st == sw.SWIGLU_OK, sw.swiglu_status_string(st)
    return (x if in_place else dx), dbias, dscale


def _noalloc(lib, x, dy, bias, scale, want_db, want_ds, in_place, dtype):
    rows, n = x.shape[0], x.shape[1] // 2
    dx = None if in_place else torch.full_like(x, float("nan"))
    dbias = torch.full((2 * n,), float("nan"), device="cuda") if want_db else None
    dscale = torch.full((rows,), float("nan"), device="cuda") if want_ds else None
    torch.cuda.synchronize()
    st = lib.swiglu_gateup_bias_scale_bwd_noalloc(
        _p(dy), n, _p(x), 2 * n, _p(bias), _p(scale), 1, _p(dx), 2 * n, _p(dbias), _p(dscale), 1,
        rows, n, _dt(dtype), int(in_place), _stream())
    assert st == sw.SWIGLU_OK, sw.swiglu_status_string(st)
    return (x if in_place else dx), dbias, dscale


def _same(a, b, what):
    if a is None:
        assert b is None
        return
    assert gu.bits_equal(a, b), f"{what} differs from the workspace entry point"


# (rows, n, dtype, want dbias, want dscale, in place): the first call is the
# 8192 x 32768 bf16 shape with both sums (48 MiB of partials), the next ones
# are smaller and leave the earlier partials in the scratch.
CALLS = [
    (8192, 32768, "bf16", True, True, False),
    (1000, 1000, "fp32", True, True, False),
    (333, 520, "bf16", True, False, True),
    (77, 4100, "fp32", False, True, True),
]


def test_noalloc_matches_workspace_entry_point():
    lib = sw.load_library()
    for i, (rows, n, dtype, want_db, want_ds, in_place) in enumerate(CALLS):
        need = lib.swiglu_gateup_bias_scale_workspace_size(rows, n, int(want_db), int(want_ds))
        _say(f"[noalloc] call {i}: rows={rows} n={n} {dtype} dbias={want_db} dscale={want_ds} "
             f"in_place={in_place} partials={need} B")
        assert need <= sw.NOALLOC_SCRATCH_BYTES
        x, dy, bias, scale = _inputs(rows, n, dtype, seed=100 + i)
        x_ref = x.clone()
        ref = _with_workspace(lib, x_ref, dy, bias, scale, want_db, want_ds, in_place, dtype)
        x_got = x.clone()
        got = _noalloc(lib, x_got, dy, bias, scale, want_db, want_ds, in_place, dtype)
        torch.cuda.synchronize()
        for a, b, what in zip(ref, got, ("dx", "dbias", "dscale")):
            _same(a, b, what)
        if not in_place:
            assert gu.bits_equal(x_got, x), "out-of-place backward touched x"
        del x, dy, bias, scale, x_ref, x_got, ref, got
    torch.cuda.synchronize()


def test_noalloc_repeated_call_same_bits():
    """The same small problem twice in a row, after a larger one has filled
    the scratch: identical results both times."""
    lib = sw.load_library()
    x, dy, bias, scale = _inputs(640, 2048, "bf16", seed=7)
    a = _noalloc(lib, x, dy, bias, scale, True, True, False, "bf16")
    b = _noalloc(lib, x, dy, bias, scale, True, True, False, "bf16")
    torch.cuda.synchronize()
    for p, q, what in zip(a, b, ("dx", "dbias", "dscale")):
        _same(p, q, what)


def test_noalloc_refuses_problems_past_the_limit():
    """16384 rows of n = 65536 with both sums need 192 MiB of partials: the
    call is refused before any launch (the buffers are real and large enough
    all the same), and the outputs keep their canaries."""
    lib = sw.load_library()
    rows, n = 16384, 65536
    need = lib.swiglu_gateup_bias_scale_workspace_size(rows, n, 1, 1)
    assert need > sw.NOALLOC_SCRATCH_BYTES
    _say(f"[noalloc] limit: rows={rows} n={n} partials={need} B")
    x = torch.zeros(rows, 2 * n, dtype=torch.bfloat16, device="cuda")
    dy = torch.zeros(rows, n, dtype=torch.bfloat16, device="cuda")
    dx = torch.zeros(rows, 2 * n, dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros(2 * n, dtype=torch.bfloat16, device="cuda")
    scale = torch.ones(rows, device="cuda")
    dbias = torch.full((2 * n,), 7.0, device="cuda")
    dscale = torch.full((rows,), 7.0, device="cuda")
    torch.cuda.synchronize()
    st = lib.swiglu_gateup_bias_scale_bwd_noalloc(
        _p(dy), n, _p(x), 2 * n, _p(bias), _p(scale), 1, _p(dx), 2 * n, _p(dbias), _p(dscale), 1,
        rows, n, sw.SWIGLU_DTYPE_BF16, 0, _stream())
    torch.cuda.synchronize()
    assert st == sw.SWIGLU_ERR_SCRATCH_LIMIT
    assert bool((dbias == 7.0).all()) and bool((dscale == 7.0).all())
    with pytest.raises(ValueError):
        sw.swiglu_gateup_bias_scale_bwd_noalloc(dy, x, dx, dbias, dscale, bias=bias, scale=scale)
    # without the sums nothing is partial, so the same size is accepted
    out, _, _ = sw.swiglu_gateup_bias_scale_bwd_noalloc(dy[:64], x[:64], dx[:64], bias=bias)
    torch.cuda.synchronize()
    assert out.data_ptr() == dx.data_ptr()
    del x, dy, dx


def test_noalloc_python_binding_matches():
    """The binding's allocation-free call against the allocating one."""
    x, dy, bias, scale = _inputs(300, 1792, "bf16", seed=9)
    ref = sw.swiglu_gateup_bias_scale_bwd(dy, x, bias, scale)
    dx = torch.empty_like(x)
    dbias = torch.empty(2 * 1792, dtype=torch.float32, device="cuda")
    dscale = torch.empty(300, dtype=torch.float32, device="cuda")
    got = sw.swiglu_gateup_bias_scale_bwd_noalloc(dy, x, dx, dbias, dscale, bias=bias, scale=scale)
    torch.cuda.synchronize()
    for a, b, what in zip(ref, got, ("dx", "dbias", "dscale")):
        _same(a, b, what)
    assert np.isfinite(gu.from_dev(dbias)).all()
