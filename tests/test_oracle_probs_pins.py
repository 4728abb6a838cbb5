"""Pins for the oracle's attention weights (oracle.probabilities): float64
torch.softmax, rows summing to one, agreement of weights x V with the forward
oracle (separate C code), causal zeros, and planted mistakes that must fail.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "attn_probs_oracle.c")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _torch_probs(q, k, scale, causal):
    s = torch.tensor(q) @ torch.tensor(k).transpose(-1, -2) * scale
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    return torch.softmax(s, -1).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_probabilities_match_torch_and_the_forward_oracle(causal):
    q, k, v = (_rand((2, 3, 33, 16), s) * 3 for s in range(3))
    w = oracle.probabilities(q, k, 0.3, causal)
    assert np.abs(w - _torch_probs(q, k, 0.3, causal)).max() <= 1e-14
    assert np.abs(w.sum(-1) - 1).max() <= 1e-14
    o, _ = oracle.attention(q, k, v, 0.3, causal)
    assert np.abs(w @ v - o).max() <= 1e-13
    if causal:
        assert np.all(np.triu(w, 1) == 0)
    rows = [32, 0, 7]
    assert np.array_equal(oracle.probabilities(q, k, 0.3, causal, rows=rows), w[..., rows, :])


MUTANTS = {
    "scale_dropped": ("wr[j] = scale * acc;", "wr[j] = acc;"),
    "diagonal_excluded": ("causal ? i : N - 1", "causal ? i - 1 : N - 1"),
    "not_normalised": ("wr[j] /= total;", "wr[j] /= 1.0;"),
    "max_kept_out": ("exp(wr[j] - top)", "exp(wr[j])"),
}


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-ffp-contract=off", "-fopenmp", str(path), "-o", str(so),
                    "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    lib.oracle_attn_probs_f64.restype = ctypes.c_int
    lib.oracle_attn_probs_f64.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
    return lib


def _passes(lib):
    for causal in (0, 1):
        q, k = _rand((1, 20, 8), 7) * 300, _rand((1, 20, 8), 8)  # scores ~1e3: exp overflows without the max
        w = np.empty((1, 20, 20))
        lib.oracle_attn_probs_f64(q.ctypes.data, k.ctypes.data, w.ctypes.data, 1, 20, 8, 0.7, causal, None, 0, 1)
        want = _torch_probs(q, k, 0.7, bool(causal))
        if not np.isfinite(w).all() or np.abs(w - want).max() > 1e-12:
            return False
    return True


def test_unmodified_source_passes(tmp_path):
    assert _passes(_build(tmp_path, "identity", "int oracle_attn_probs_f64", "int oracle_attn_probs_f64"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    assert not _passes(_build(tmp_path, name, *MUTANTS[name])), name
