"""The kernels under HIP graph capture (needs an MI355X).

Training loops capture their steps in graphs; the library's launches go to
the caller's stream and allocate nothing, so they can be captured. Each
test captures once, then replays several times with new inputs copied into
the captured buffers, eager work and synchronizations in between, and
checks every replay bitwise against the eager result on the same inputs.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import swiglu_activation_amd as sw
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
REPLAYS = 5


def _bf16(rng, shape, scale=1.0):
    return gu.to_dev(oracle.round_f64_to_bf16_bits(rng.standard_normal(shape) * scale), "bf16")


def test_gateup_fwd_bwd_replays_match_eager():
    rows, n = 300, 1100
    print(f"[graph] gate-up fwd + bwd (out of place and in place), rows {rows} n {n}", flush=True)
    rng = np.random.default_rng(60)
    xs, dys = _bf16(rng, (rows, 2 * n), 3.0), _bf16(rng, (rows, n))
    ys, dxs = torch.empty(rows, n, dtype=torch.bfloat16, device="cuda"), torch.empty_like(xs)
    xi = xs.clone()                                   # overwritten in place by the graph
    sw.swiglu_gateup_fwd(xs, ys)                      # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw.swiglu_gateup_fwd(xs, ys)
        sw.swiglu_gateup_bwd(dys, xs, dxs)
        sw.swiglu_gateup_bwd(dys, xi, in_place=True)
    for r in range(REPLAYS):
        x, dy = _bf16(rng, (rows, 2 * n), 3.0), _bf16(rng, (rows, n))
        xs.copy_(x)
        xi.copy_(x)
        dys.copy_(dy)
        y_e = sw.swiglu_gateup_fwd(x)
        dx_e = sw.swiglu_gateup_bwd(dy, x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert gu.bits_equal(ys, y_e), r
        assert gu.bits_equal(dxs, dx_e), r
        assert gu.bits_equal(xi, dx_e), r


def test_bias_scale_backward_with_sums_replays_match_eager():
    rows, n = 515, 2048
    print(f"[graph] bias/scale bwd with dbias and dscale, rows {rows} n {n}", flush=True)
    rng = np.random.default_rng(61)
    xs, dys = _bf16(rng, (rows, 2 * n), 2.0), _bf16(rng, (rows, n))
    bias = _bf16(rng, (2 * n,), 0.5)
    scale = torch.from_numpy(rng.uniform(0.05, 1.0, rows).astype(np.float32)).cuda()
    ws = torch.empty(sw.swiglu_gateup_bias_scale_workspace_size(rows, n, True, True),
                     dtype=torch.uint8, device="cuda")
    sw.swiglu_gateup_bias_scale_bwd(dys, xs, bias, scale, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ys = sw.swiglu_gateup_bias_scale_fwd(xs, bias, scale)
        dxs, dbs, dss = sw.swiglu_gateup_bias_scale_bwd(dys, xs, bias, scale, workspace=ws)
    for r in range(REPLAYS):
        x, dy = _bf16(rng, (rows, 2 * n), 2.0), _bf16(rng, (rows, n))
        xs.copy_(x)
        dys.copy_(dy)
        y_e = sw.swiglu_gateup_bias_scale_fwd(x, bias, scale)
        dx_e, db_e, ds_e = sw.swiglu_gateup_bias_scale_bwd(dy, x, bias, scale)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert gu.bits_equal(ys, y_e), r
        assert gu.bits_equal(dxs, dx_e), r
        assert torch.equal(dbs.view(torch.int32), db_e.view(torch.int32)), r
        assert torch.equal(dss.view(torch.int32), ds_e.view(torch.int32)), r


def test_fc1_replays_match_eager():
    m, n, k = 520, 384, 640
    print(f"[graph] fc1 + SwiGLU m {m} n {n} k {k}", flush=True)
    rng = np.random.default_rng(62)
    a_s, w_s = _bf16(rng, (m, k)), _bf16(rng, (2 * n, k), k ** -0.5)
    y_s = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    sw.swiglu_fc1_fwd(a_s, w_s, y_s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw.swiglu_fc1_fwd(a_s, w_s, y_s)
    for r in range(REPLAYS):
        a, w = _bf16(rng, (m, k)), _bf16(rng, (2 * n, k), k ** -0.5)
        a_s.copy_(a)
        w_s.copy_(w)
        y_e = sw.swiglu_fc1_fwd(a, w)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert gu.bits_equal(y_s, y_e), r


def test_fc1_pool_with_explicit_workspace_replays_match_eager():
    """A launch large enough for the tile pool (128 feature tiles x 32 token
    tiles), captured with a caller's workspace: the last pool workgroup
    clears the queue counters inside every replay, so each replay matches
    an eager call with no workspace, and the workspace is zero after each."""
    m, n, k = 8192, 16384, 64
    print(f"[graph] fc1 pool m {m} n {n} k {k}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(63)
    a_s = torch.randn(m, k, device="cuda", generator=gen).bfloat16()
    w_s = (torch.randn(2 * n, k, device="cuda", generator=gen) / k ** 0.5).bfloat16()
    y_s = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(sw.swiglu_fc1_workspace_size(), dtype=torch.uint8, device="cuda")
    sw.swiglu_fc1_fwd(a_s, w_s, y_s, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw.swiglu_fc1_fwd(a_s, w_s, y_s, workspace=ws)
    for r in range(REPLAYS):
        a_s.copy_(torch.randn(m, k, device="cuda", generator=gen).bfloat16())
        y_e = sw.swiglu_fc1_fwd(a_s, w_s, workspace=False)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert gu.bits_equal(y_s, y_e), r
        assert int(ws.count_nonzero()) == 0, r
