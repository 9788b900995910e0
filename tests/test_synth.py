"""The seeded input generator (no GPU)."""

import numpy as np

import oracle
import synth


def test_blocks_are_independent_of_range():
    w = synth.WORKLOADS["inplace_tp_bf16_t8192_n1792"]
    full = synth.make_x(w, 0, 1500)
    part = synth.make_x(w, 600, 1100, threads=1)
    assert np.array_equal(full[600:1100], part)
    assert np.array_equal(synth.make_dy(w, 0, 1500)[1000:1200], synth.make_dy(w, 1000, 1200))


def test_deterministic_and_seed_dependent():
    w = synth.WORKLOADS[synth.SMALL]
    a, b = synth.make_x(w), synth.make_x(w)
    assert a.dtype == np.float32 and a.shape == (64, 256)
    assert np.array_equal(a, b)
    assert not np.array_equal(synth.make_dy(w), a[:, :128])
    w2 = synth.WORKLOADS["dense_bf16_s2048_b4_n4096"]
    assert synth.make_x(w2, 0, 4).dtype == np.uint16


def test_input_rounding_is_nearest_even_bf16():
    """The generator's own float64 -> bf16 rounding agrees with the oracle's
    independent implementation on the value ranges it draws."""
    rng = np.random.default_rng(9)
    v = np.concatenate([rng.standard_normal(200_000), rng.uniform(-30, 30, 200_000), [0.0, -0.0]])
    assert np.array_equal(synth._f64_to_bf16_bits_inputs(v), oracle.round_f64_to_bf16_bits(v))


def test_distributions():
    w = synth.WORKLOADS["odd_fp32_s4096_b1_n11008"]
    x = synth.make_x(w, 0, 512).astype(np.float64)
    g, u = x[:, :w.n], x[:, w.n:]
    sat = np.abs(g) > 6
    assert 0.08 < sat.mean() < 0.11                 # about 1 in 10 from U[-30, 30)
    assert np.abs(g).max() <= 30.0
    assert abs(u.std() - np.sqrt(2.0)) < 0.01        # variance 2
    w3 = synth.WORKLOADS[synth.HEADLINE]
    b = oracle.bf16_bits_to_f64(synth.make_x(w3, 0, 64))
    assert abs(b.mean()) < 0.01 and abs(b.std() - 1) < 0.01


def test_workload_shapes():
    W = synth.WORKLOADS
    assert (W[synth.HEADLINE].rows, W[synth.HEADLINE].n) == (8192, 32768)
    assert (W["odd_fp32_s4096_b1_n11008"].rows, W["odd_fp32_s4096_b1_n11008"].n) == (4096, 11008)
    assert W["inplace_tp_bf16_t8192_n1792"].n == 1792
    assert W[synth.SMALL].rows == 64
    rows = synth.sample_rows(W[synth.HEADLINE], 64)
    assert rows[0] == 0 and rows[-1] == 8191 and len(rows) == 64
