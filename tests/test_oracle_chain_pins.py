"""Pins for the oracle's elementwise chain (oracle.elementwise_chain):
hand-computed values, the activation's definition (negatives to zero,
positives unchanged), broadcasting of the bias along rows, and float64 torch
composed from its own primitives."""
import numpy as np
import torch

import oracle


def test_hand_values():
    x = np.array([[1.0, -2.0, 0.5, 3.0], [-1.0, 0.0, 2.0, -0.25]])
    b = np.array([0.5, 1.0, -2.0, 0.0])
    y, t1, t2 = oracle.elementwise_chain(x, 2.0, b)
    assert np.array_equal(t1, [[2.0, -4.0, 1.0, 6.0], [-2.0, 0.0, 4.0, -0.5]])
    assert np.array_equal(t2, [[2.5, -3.0, -1.0, 6.0], [-1.5, 1.0, 2.0, -0.5]])
    assert np.array_equal(y, [[2.5, 0.0, 0.0, 6.0], [0.0, 1.0, 2.0, 0.0]])


def test_activation_and_broadcast():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 16))
    b = rng.standard_normal(16)
    y, _, t2 = oracle.elementwise_chain(x, -0.75, b)
    assert np.all(y >= 0) and np.array_equal(y[t2 > 0], t2[t2 > 0]) and np.all(y[t2 <= 0] == 0)
    # the same bias element reaches every row of its column
    y2, _, _ = oracle.elementwise_chain(x[3:4], -0.75, b)
    assert np.array_equal(y2[0], y[3])


def test_matches_float64_torch():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(33, 40, generator=g, dtype=torch.float64)
    b = torch.randn(40, generator=g, dtype=torch.float64)
    y, _, _ = oracle.elementwise_chain(x.numpy(), 1.5, b.numpy())
    assert np.array_equal(y, torch.relu(x * 1.5 + b).numpy())


def test_scale_is_taken_in_float32():
    # The kernels take scale as a float32; the oracle uses that same value.
    y, t1, _ = oracle.elementwise_chain(np.ones((1, 8)), 0.1, np.zeros(8))
    assert t1[0, 0] == float(np.float32(0.1)) and t1[0, 0] != 0.1


MUTANTS = {
    "bias_before_scale": ("t2 = t1 + b64[None, :]", "t2 = float(np.float32(scale)) * (x64 + b64[None, :])"),
    "no_activation": ("y = np.where(t2 > 0.0, t2, 0.0)", "y = t2"),
    "bias_along_rows": ("t2 = t1 + b64[None, :]", "t2 = t1 + b64[:, None][: x64.shape[0]]"),
    "leaky_activation": ("y = np.where(t2 > 0.0, t2, 0.0)", "y = np.where(t2 > 0.0, t2, 0.01 * t2)"),
}


def _mutant(old, new):
    import inspect
    src = inspect.getsource(oracle.elementwise_chain)
    assert src.count(old) == 1
    ns = {"np": np, "_as_f64": oracle._as_f64}
    exec(src.replace(old, new), ns)
    return ns["elementwise_chain"]


def _passes(fn):
    x = np.array([[1.0, -2.0, 0.5, 3.0], [-1.0, 0.0, 2.0, -0.25], [4.0, 1.0, -1.0, 2.0], [0.0, 0.0, 0.0, 1.0]])
    b = np.array([0.5, 1.0, -2.0, 0.0])
    try:
        y, _, _ = fn(x, 2.0, b)
    except Exception:
        return False
    want = np.maximum(2.0 * x + b[None, :], 0.0)
    return y.shape == want.shape and np.array_equal(y, want)


def test_unmodified_chain_source_passes():
    assert _passes(_mutant("y = np.where", "y = np.where"))


def test_planted_chain_mistakes_are_caught():
    for name, (old, new) in MUTANTS.items():
        assert not _passes(_mutant(old, new)), name
