"""fc1 projection with the SwiGLU epilogue vs the oracle (needs an MI355X).

Bar. Inputs are bf16, products exact in fp32, sums accumulated in fp32 by
the matrix cores in an unspecified order, so each accumulator D obeys
|D - D_exact| <= E = k * 2^-24 * (|A| |W|^T) (the float64 sum of magnitudes).
The epilogue then forms silu(g) u in fp32 and rounds once to bf16, so
    |y - y_ref| <= 2 ulp_bf16(y_ref) + |silu'(g)| |u| E_g + |silu(g)| E_u
(+ |E_g E_u| terms far below these), where g, u are the exact products. The
product written to x_out obeys |x - x_ref| <= 1 ulp_bf16(x_ref) + E.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import swiglu_activation_amd as sw
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _bf16_ulp(v):
    """Spacing of the bf16 grid at |v| (subnormal spacing below 2^-126)."""
    a = np.abs(v)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def _case(m, n, k, seed, scale_a=1.0):
    rng = np.random.default_rng(seed)
    a = oracle.round_f64_to_bf16_bits(rng.standard_normal((m, k)) * scale_a)
    w = oracle.round_f64_to_bf16_bits(rng.standard_normal((2 * n, k)) / np.sqrt(k))
    return a, w


def _check(a_h, w_h, y, x=None):
    af, wf = oracle.widen(a_h, "bf16"), oracle.widen(w_h, "bf16")
    n, k = wf.shape[0] // 2, wf.shape[1]
    xref = oracle.oracle_fc1(af, wf)
    yref = oracle.oracle_fwd(xref)
    E = k * 2.0 ** -24 * (np.abs(af) @ np.abs(wf).T)
    g, u = xref[:, :n], xref[:, n:]
    s = oracle.sigmoid(g)
    bound = (2 * _bf16_ulp(yref) + np.abs(oracle.silu_grad(g)) * np.abs(u) * E[:, :n]
             + np.abs(g * s) * E[:, n:] + E[:, :n] * E[:, n:])
    got = oracle.bf16_bits_to_f64(gu.from_dev(y))
    err = np.abs(got - yref)
    worst = float(np.max(err / bound))
    print(f"    y: {yref.size} elements, worst {worst:.3g} of the bar", flush=True)
    assert np.all(err <= bound), worst
    if x is not None:
        gx = oracle.bf16_bits_to_f64(gu.from_dev(x))
        bx = _bf16_ulp(xref) + E
        wx = float(np.max(np.abs(gx - xref) / bx))
        print(f"    x: {xref.size} elements, worst {wx:.3g} of the bar", flush=True)
        assert np.all(np.abs(gx - xref) <= bx), wx


@pytest.mark.parametrize("m,n,k", [(128, 128, 64), (256, 256, 512), (300, 192, 320),
                                   (1, 64, 64), (1000, 1792, 1024), (4096, 512, 4096),
                                   (260, 320, 384), (192, 128, 192), (96, 64, 1984),
                                   (64, 128, 65536)])
def test_fc1_swiglu_parity(m, n, k):
    """Ragged token counts (300, 1, 1000, 260), a feature count that leaves a
    half-empty 128-wide tile (192, 1792, 320), and long k (up to 65536). The
    k loop is unrolled over periods of 6 k tiles and skips the first
    (-k/64) mod 6 slots; these k cover every count of skipped slots: 64 and
    1984 skip 5, 512 skips 4, 192 skips 3, 1024, 4096 and 65536 skip 2, 320
    skips 1, 384 skips none."""
    print(f"[fc1] m={m} n={n} k={k}", flush=True)
    a_h, w_h = _case(m, n, k, seed=m + n + k)
    a, w = gu.to_dev(a_h, "bf16"), gu.to_dev(w_h, "bf16")
    y, x = sw.swiglu_fc1_fwd(a, w, x_out=True)
    torch.cuda.synchronize()
    _check(a_h, w_h, y, x)
    # the product written for the backward feeds the elementwise kernel to the same y
    y2 = sw.swiglu_gateup_fwd(x)
    torch.cuda.synchronize()
    assert y2.shape == y.shape


def test_fc1_swiglu_3d_input_and_strided_output():
    a_h, w_h = _case(2 * 96, 256, 256, seed=7)
    a = gu.to_dev(a_h, "bf16").reshape(2, 96, 256)
    w = gu.to_dev(w_h, "bf16")
    yb = torch.full((2 * 96, 256 + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = yb[:, :256]
    sw.swiglu_fc1_fwd(a.reshape(192, 256), w, y)
    y3 = sw.swiglu_fc1_fwd(a, w)
    torch.cuda.synchronize()
    assert y3.shape == (2, 96, 256)
    assert gu.bits_equal(y3.reshape(192, 256), y)
    assert torch.isnan(yb[:, 256:]).all()
    _check(a_h, w_h, y)


def test_fc1_deterministic():
    a_h, w_h = _case(512, 512, 1024, seed=8)
    a, w = gu.to_dev(a_h, "bf16"), gu.to_dev(w_h, "bf16")
    y1 = sw.swiglu_fc1_fwd(a, w)
    y2 = sw.swiglu_fc1_fwd(a, w)
    torch.cuda.synchronize()
    assert gu.bits_equal(y1, y2)


def test_fc1_argument_errors():
    a = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(128, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        sw.swiglu_fc1_fwd(a.float(), w.float())                          # bf16 only
    with pytest.raises(ValueError):
        sw.swiglu_fc1_fwd(a[:, :32], w[:, :32])                          # k not a multiple of 64
    with pytest.raises(ValueError):
        sw.swiglu_fc1_fwd(a, torch.zeros(96, 64, dtype=torch.bfloat16, device="cuda"))  # n = 48
    with pytest.raises(ValueError):
        sw.swiglu_fc1_fwd(a, w, a[:, :64])                               # y overlaps a
    with pytest.raises(ValueError):
        sw.swiglu_fc1_fwd(a, w, torch.empty(8, 64, device="cuda"))      # float32 y
    with pytest.raises(ValueError):
        sw.swiglu_fc1_fwd(a, w, x_out=torch.empty(8, 128, device="cuda"))  # float32 x_out


@pytest.mark.parametrize("hidden,n", [(4096, 4096), (8192, 32768)])
def test_fc1_full_size_sampled(hidden, n):
    """The benchmark's shapes and launch (8192 tokens, one call writing y,
    then one also writing the product). Inputs are drawn on the device with
    a seeded torch generator (N(0,1) activations, N(0,1/hidden) weights,
    rounded to bf16); y and the product are compared with the oracle on a
    64 x 64 block of sampled (token, feature) pairs that includes the first
    and last rows and the edges of the workgroup tiles."""
    m = 8192
    print(f"[fc1 full] tokens {m} hidden {hidden} n {n}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(hidden + n)
    a = torch.randn(m, hidden, device="cuda", generator=gen).bfloat16()
    w = (torch.randn(2 * n, hidden, device="cuda", generator=gen) / hidden ** 0.5).bfloat16()
    y = sw.swiglu_fc1_fwd(a, w)
    y2, x = sw.swiglu_fc1_fwd(a, w, x_out=True)
    y3 = sw.swiglu_fc1_fwd(a, w, workspace=False)      # one workgroup per tile
    torch.cuda.synchronize()
    assert gu.bits_equal(y, y2) and gu.bits_equal(y, y3)
    rng = np.random.default_rng(hidden + n)
    toks = np.unique(np.concatenate([[0, 1, 255, 256, 511, m - 1],
                                     rng.choice(m, 58, replace=False)]))
    feats = np.unique(np.concatenate([[0, 63, 64, 127, 128, n - 1],
                                      rng.choice(n, 58, replace=False)]))
    ti = torch.from_numpy(toks).cuda()
    fi = torch.from_numpy(feats).cuda()
    a_s = gu.from_dev(a[ti])
    w_s = gu.from_dev(torch.cat([w[fi], w[fi + n]]))
    y_s = y[ti][:, fi]
    x_s = torch.cat([x[ti][:, fi], x[ti][:, fi + n]], dim=1)
    _check(a_s, w_s, y_s, x_s)
    del a, w, y, y2, y3, x


@pytest.mark.parametrize("m", [8192, 8192 + 100])
def test_fc1_tile_pool(m):
    """A launch of at least 16 tiles per CU (128 feature tiles x 32 or 33
    token tiles) ends on a pool of tiles that workgroups take through the
    workspace's queues. Three calls in a row on one workspace: y and the
    product are the same bits as with one workgroup per tile, the workspace
    is all zero after each call, and y matches the oracle on sampled pairs
    from the pool's tiles (the last quarter of the launch order: features
    12288 and up) and from the fixed ones."""
    n, k = 16384, 128
    print(f"[fc1 pool] m={m} n={n} k={k}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(m)
    a = torch.randn(m, k, device="cuda", generator=gen).bfloat16()
    w = (torch.randn(2 * n, k, device="cuda", generator=gen) / k ** 0.5).bfloat16()
    y_fixed, x_fixed = sw.swiglu_fc1_fwd(a, w, x_out=True, workspace=False)
    ws = torch.zeros(sw.swiglu_fc1_workspace_size(), dtype=torch.uint8, device="cuda")
    for call in range(3):
        y, x = sw.swiglu_fc1_fwd(a, w, x_out=True, workspace=ws)
        torch.cuda.synchronize()
        print(f"    call {call}", flush=True)
        assert gu.bits_equal(y, y_fixed) and gu.bits_equal(x, x_fixed)
        assert int(ws.count_nonzero()) == 0
    rng = np.random.default_rng(m)
    toks = np.unique(np.concatenate([[0, 255, 256, m - 1], rng.choice(m, 28, replace=False)]))
    feats = np.unique(np.concatenate([[0, 12287, 12288, n - 1],
                                      rng.choice(n, 28, replace=False)]))
    ti = torch.from_numpy(toks).cuda()
    fi = torch.from_numpy(feats).cuda()
    _check(gu.from_dev(a[ti]), gu.from_dev(torch.cat([w[fi], w[fi + n]])), y[ti][:, fi])


def test_fc1_two_streams():
    """Launches on two streams at once, each with the binding's own
    workspace for its stream: both equal the launch with one workgroup per
    tile."""
    m, n, k = 8192, 16384, 64
    print(f"[fc1 streams] m={m} n={n} k={k}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(3)
    a = torch.randn(m, k, device="cuda", generator=gen).bfloat16()
    w = (torch.randn(2 * n, k, device="cuda", generator=gen) / k ** 0.5).bfloat16()
    y_fixed = sw.swiglu_fc1_fwd(a, w, workspace=False)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ys = []
    for rep in range(2):
        with torch.cuda.stream(s1):
            y1 = sw.swiglu_fc1_fwd(a, w)
        with torch.cuda.stream(s2):
            y2 = sw.swiglu_fc1_fwd(a, w)
        ys += [y1, y2]
    torch.cuda.synchronize()
    for y in ys:
        assert gu.bits_equal(y, y_fixed)


def test_fc1_strided_operands():
    """a and w as column slices of wider buffers (row strides k + 64 and
    k + 128), the product written into a wider buffer whose extra columns
    must stay untouched."""
    m, n, k = 384, 256, 512
    print(f"[fc1 strided] m={m} n={n} k={k}", flush=True)
    a_h, w_h = _case(m, n, k, seed=9)
    ab = torch.zeros(m, k + 64, dtype=torch.bfloat16, device="cuda")
    ab[:, :k] = gu.to_dev(a_h, "bf16")
    wb = torch.zeros(2 * n, k + 128, dtype=torch.bfloat16, device="cuda")
    wb[:, :k] = gu.to_dev(w_h, "bf16")
    xb = torch.full((m, 2 * n + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    y, x = sw.swiglu_fc1_fwd(ab[:, :k], wb[:, :k], x_out=xb[:, :2 * n])
    torch.cuda.synchronize()
    assert torch.isnan(xb[:, 2 * n:]).all()
    _check(a_h, w_h, y, x)
    y_dense = sw.swiglu_fc1_fwd(gu.to_dev(a_h, "bf16"), gu.to_dev(w_h, "bf16"))
    torch.cuda.synchronize()
    assert gu.bits_equal(y, y_dense)


@pytest.mark.parametrize("m,n,k", [(96, 128, 65536), (300, 192, 2496)])
def test_fc1_exact_sums(m, n, k):
    """Inputs chosen so that fp32 accumulation is exact in any order: a in
    {-1, 0, 1}, w in {-1/8, 0, 1/8}, so every product is a multiple of 1/8
    and every partial sum stays below 2^24 / 8 in magnitude. A missing,
    repeated or misplaced k tile then shows as a wrong value, which the
    fp32-accumulation bound of the other tests (k 2^-24 |A||W|, about 0.4
    at k = 65536) would not catch. The product must equal the oracle's
    nearest-even bf16 rounding of the exact sums bit for bit, and y must be
    within 2 bf16 ulp of the oracle's correctly rounded value.
    k = 65536 runs 1024 k tiles (two skipped slots); 2496 runs 39 (three)."""
    print(f"[fc1 exact] m={m} n={n} k={k}", flush=True)
    rng = np.random.default_rng(m + k)
    a_h = oracle.round_f64_to_bf16_bits(rng.integers(-1, 2, (m, k)).astype(np.float64))
    w_h = oracle.round_f64_to_bf16_bits(rng.integers(-1, 2, (2 * n, k)).astype(np.float64) / 8)
    a, w = gu.to_dev(a_h, "bf16"), gu.to_dev(w_h, "bf16")
    y, x = sw.swiglu_fc1_fwd(a, w, x_out=True)
    torch.cuda.synchronize()
    af, wf = oracle.widen(a_h, "bf16"), oracle.widen(w_h, "bf16")
    xref = oracle.oracle_fc1(af, wf)
    assert np.max(np.abs(xref)) * 8 < 2 ** 24            # every partial sum is exact in fp32
    assert np.array_equal(gu.from_dev(x), oracle.round_f64_to_bf16_bits(xref))
    yref = oracle.round_f64_to_bf16_bits(oracle.oracle_fwd(xref))
    dist = oracle.bf16_ulp_distance(gu.from_dev(y), yref)
    print(f"    y: max {int(dist.max())} ulp over {dist.size}", flush=True)
    assert int(dist.max()) <= 2
