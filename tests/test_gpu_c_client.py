"""The C ABI from a plain C program (needs an MI355X).

swiglu_activation_amd/examples/c_abi_client.c links libswiglu_gateup.so with
no Python or torch and calls every entry point of swiglu_gateup.h on one HIP
stream, including some argument errors. These tests give it seeded inputs
through files, run it as a child process, and check its outputs: the packed
and two-tensor forward and backward against the oracle, the bias / scale and
fc1 entry points bit for bit against the Python binding on the same inputs
(the binding's results are checked against the oracle in their own tests).
"""

from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import swiglu_activation_amd as sw
from swiglu_activation_amd import build
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run(*args):
    if not os.path.exists(build.CLIENT):
        pytest.fail("the C client is not built (swiglu_activation_amd.build.build())")
    res = subprocess.run([build.CLIENT, *map(str, args)], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stderr
    assert "c_abi_client: ok" in res.stdout


def _inputs(rows, n, seed):
    rng = np.random.default_rng(seed)
    x_h = oracle.round_f64_to_bf16_bits(np.concatenate(
        [rng.standard_normal((rows, n)) * 3, rng.standard_normal((rows, n))], 1))
    dy_h = oracle.round_f64_to_bf16_bits(rng.standard_normal((rows, n)))
    return x_h, dy_h


@pytest.mark.parametrize("mode", ["gateup", "silu_mul"])
@pytest.mark.parametrize("rows,n", [(333, 2048), (64, 1001)])
def test_c_client_matches_oracle(tmp_path, mode, rows, n):
    print(f"[c client {mode}] rows={rows} n={n}", flush=True)
    x_h, dy_h = _inputs(rows, n, rows + n)
    f = {k: str(tmp_path / f"{k}.bin") for k in ("x", "dy", "y", "dx", "dxi")}
    x_h.tofile(f["x"])
    dy_h.tofile(f["dy"])
    _run(mode, rows, n, f["x"], f["dy"], f["y"], f["dx"], f["dxi"])
    y = np.fromfile(f["y"], dtype=np.uint16).reshape(rows, n)
    dx = np.fromfile(f["dx"], dtype=np.uint16).reshape(rows, 2 * n)
    dxi = np.fromfile(f["dxi"], dtype=np.uint16).reshape(rows, 2 * n)
    assert np.array_equal(dx, dxi)                    # in place: the same bits
    xf, dyf = oracle.widen(x_h, "bf16"), oracle.widen(dy_h, "bf16")
    for got, ref, what in ((y, oracle.oracle_fwd(xf), "fwd"), (dx, oracle.oracle_bwd(xf, dyf), "bwd")):
        st = gu.compare(got, ref, "bf16", what)
        print("   ", st, flush=True)
        assert st.ok(), str(st)


def test_c_client_bias_scale_matches_binding(tmp_path):
    rows, n = 515, 2048
    print(f"[c client bias_scale] rows={rows} n={n}", flush=True)
    x_h, dy_h = _inputs(rows, n, 71)
    rng = np.random.default_rng(72)
    b_h = oracle.round_f64_to_bf16_bits(rng.standard_normal(2 * n) * 0.5)
    s_h = rng.uniform(0.05, 1.0, rows).astype(np.float32)
    f = {k: str(tmp_path / f"{k}.bin")
         for k in ("x", "dy", "b", "s", "y", "dx", "db", "ds")}
    for k, a in (("x", x_h), ("dy", dy_h), ("b", b_h), ("s", s_h)):
        a.tofile(f[k])
    _run("bias_scale", rows, n, f["x"], f["dy"], f["b"], f["s"], f["y"], f["dx"], f["db"], f["ds"])
    x, dy, b = gu.to_dev(x_h, "bf16"), gu.to_dev(dy_h, "bf16"), gu.to_dev(b_h, "bf16")
    s = torch.from_numpy(s_h).cuda()
    y = sw.swiglu_gateup_bias_scale_fwd(x, b, s)
    dx, db, ds = sw.swiglu_gateup_bias_scale_bwd(dy, x, b, s)
    torch.cuda.synchronize()
    assert np.array_equal(np.fromfile(f["y"], dtype=np.uint16).reshape(rows, n), gu.from_dev(y))
    assert np.array_equal(np.fromfile(f["dx"], dtype=np.uint16).reshape(rows, 2 * n),
                          gu.from_dev(dx))
    assert np.array_equal(np.fromfile(f["db"], dtype=np.float32).view(np.uint32),
                          db.cpu().numpy().view(np.uint32))
    assert np.array_equal(np.fromfile(f["ds"], dtype=np.float32).view(np.uint32),
                          ds.cpu().numpy().view(np.uint32))


def test_c_client_fc1_matches_binding(tmp_path):
    m, n, k = 300, 192, 320
    print(f"[c client fc1] m={m} n={n} k={k}", flush=True)
    rng = np.random.default_rng(73)
    a_h = oracle.round_f64_to_bf16_bits(rng.standard_normal((m, k)))
    w_h = oracle.round_f64_to_bf16_bits(rng.standard_normal((2 * n, k)) / np.sqrt(k))
    f = {key: str(tmp_path / f"{key}.bin") for key in ("a", "w", "y", "x")}
    a_h.tofile(f["a"])
    w_h.tofile(f["w"])
    _run("fc1", m, n, k, f["a"], f["w"], f["y"], f["x"])
    y, x = sw.swiglu_fc1_fwd(gu.to_dev(a_h, "bf16"), gu.to_dev(w_h, "bf16"), x_out=True)
    torch.cuda.synchronize()
    assert np.array_equal(np.fromfile(f["y"], dtype=np.uint16).reshape(m, n), gu.from_dev(y))
    assert np.array_equal(np.fromfile(f["x"], dtype=np.uint16).reshape(m, 2 * n), gu.from_dev(x))
