"""The C ABI from a plain C program (needs an MI355X).

swiglu_activation_amd/examples/c_abi_client.c links libswiglu_gateup.so with
no Python or torch: it reads x and dy, runs the forward, the out-of-place
and the in-place backward on one HIP stream, checks four argument errors,
and writes the results. This test gives it seeded inputs through files, runs
it as a child process, and compares its outputs with the oracle.
"""

from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
from swiglu_activation_amd import build
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,n", [(333, 2048), (64, 1001)])
def test_c_client_matches_oracle(tmp_path, rows, n):
    print(f"[c client] rows={rows} n={n}", flush=True)
    if not os.path.exists(build.CLIENT):
        pytest.fail("the C client is not built (swiglu_activation_amd.build.build())")
    rng = np.random.default_rng(rows + n)
    x_h = oracle.round_f64_to_bf16_bits(np.concatenate(
        [rng.standard_normal((rows, n)) * 3, rng.standard_normal((rows, n))], 1))
    dy_h = oracle.round_f64_to_bf16_bits(rng.standard_normal((rows, n)))
    files = {k: str(tmp_path / f"{k}.bin") for k in ("x", "dy", "y", "dx", "dxi")}
    x_h.tofile(files["x"])
    dy_h.tofile(files["dy"])
    res = subprocess.run([build.CLIENT, str(rows), str(n), files["x"], files["dy"], files["y"],
                          files["dx"], files["dxi"]], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert "c_abi_client: ok" in res.stdout
    y = np.fromfile(files["y"], dtype=np.uint16).reshape(rows, n)
    dx = np.fromfile(files["dx"], dtype=np.uint16).reshape(rows, 2 * n)
    dxi = np.fromfile(files["dxi"], dtype=np.uint16).reshape(rows, 2 * n)
    assert np.array_equal(dx, dxi)                    # in place: the same bits
    xf, dyf = oracle.widen(x_h, "bf16"), oracle.widen(dy_h, "bf16")
    for got, ref, what in ((y, oracle.oracle_fwd(xf), "fwd"), (dx, oracle.oracle_bwd(xf, dyf), "bwd")):
        st = gu.compare(got, ref, "bf16", what)
        print("   ", st, flush=True)
        assert st.ok(), str(st)
