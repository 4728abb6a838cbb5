"""Pins for the oracle's masked / biased attention (oracle.attention_masked):
reduction to the plain oracle (separate C code), float64 torch.softmax with an
explicit mask and bias, closed forms (a zero-width window gives o_i = v_i; a
per-row constant bias shifts lse only; an all -inf row gives o = 0 and
lse = -inf), and planted mistakes that must fail.
"""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "attn_masked_oracle.c")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _allowed(N, causal, wl, wr):
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    a = np.ones((N, N), dtype=bool)
    if causal:
        a &= j <= i
    if wl >= 0:
        a &= j >= i - wl
    if wr >= 0:
        a &= j <= i + wr
    return a


def _torch_ref(q, k, v, scale, causal, wl, wr, bias):
    s = torch.tensor(q) @ torch.tensor(k).transpose(-1, -2) * scale
    if bias is not None:
        s = s + torch.tensor(bias)
    s = s.masked_fill(~torch.tensor(_allowed(q.shape[-2], causal, wl, wr)), float("-inf"))
    return (torch.softmax(s, -1) @ torch.tensor(v)).numpy(), torch.logsumexp(s, -1).numpy()


def test_reduces_to_the_plain_oracle():
    q, k, v = (_rand((2, 3, 37, 16), s) for s in range(3))
    for causal in (False, True):
        o, lse = oracle.attention_masked(q, k, v, 0.25, causal)
        o2, lse2 = oracle.attention(q, k, v, 0.25, causal)
        assert np.abs(o - o2).max() <= 1e-13 and np.abs(lse - lse2).max() <= 1e-13


BIAS_SHAPES = [None, (1, 1), (2, 1), (1, 3), (2, 3)]


@pytest.mark.parametrize("bshape", BIAS_SHAPES)
@pytest.mark.parametrize("causal,wl,wr", [(False, -1, -1), (False, 0, 0), (False, 3, -1), (False, -1, 2),
                                         (False, 5, 5), (True, -1, -1), (True, 4, -1), (True, 0, 0)])
def test_matches_float64_torch(bshape, causal, wl, wr):
    B, H, N, d = 2, 3, 29, 8
    q, k, v = (_rand((B, H, N, d), 10 + s) for s in range(3))
    bias = None
    if bshape is not None:
        bias = _rand(bshape + (N, N), 20) * 2
        # remove some keys, never a row's diagonal (no row becomes empty)
        drop = np.random.default_rng(21).random(bias.shape) < 0.2
        drop &= ~np.eye(N, dtype=bool)[None, None]
        bias[drop] = -np.inf
    o, lse = oracle.attention_masked(q, k, v, 0.4, causal, wl, wr, bias)
    o_t, lse_t = _torch_ref(q, k, v, 0.4, causal, wl, wr, bias)
    assert np.abs(o - o_t).max() <= 1e-12
    assert np.abs(lse - lse_t).max() <= 1e-12


def test_zero_width_window_returns_v():
    q, k, v = (_rand((1, 2, 15, 4), 30 + s) for s in range(3))
    bias = _rand((1, 2, 15, 15), 33)
    o, lse = oracle.attention_masked(q, k, v, 0.7, False, 0, 0, bias)
    assert np.abs(o - v).max() <= 1e-15
    diag = 0.7 * np.einsum("bhnd,bhnd->bhn", q, k) + np.diagonal(bias, axis1=2, axis2=3)
    assert np.abs(lse - diag).max() <= 1e-13


def test_row_constant_bias_shifts_lse_only():
    q, k, v = (_rand((2, 2, 21, 8), 40 + s) for s in range(3))
    c = _rand((1, 2, 21, 1), 44) * 5
    o0, l0 = oracle.attention_masked(q, k, v, 0.3, True, 6, -1)
    o1, l1 = oracle.attention_masked(q, k, v, 0.3, True, 6, -1, np.broadcast_to(c, (1, 2, 21, 21)))
    assert np.abs(o1 - o0).max() <= 1e-13
    assert np.abs(l1 - (l0 + c[..., 0])).max() <= 1e-12


def test_empty_row_gives_zero_and_minus_inf():
    q, k, v = (_rand((1, 1, 9, 4), 50 + s) for s in range(3))
    bias = np.zeros((1, 1, 9, 9))
    bias[0, 0, 4, :] = -np.inf
    o, lse = oracle.attention_masked(q, k, v, 0.5, False, -1, -1, bias)
    assert np.all(o[0, 0, 4] == 0) and lse[0, 0, 4] == -np.inf
    assert np.isfinite(o).all() and np.isfinite(np.delete(lse[0, 0], 4)).all()


def test_window_wider_than_the_sequence_is_no_window():
    q, k, v = (_rand((1, 2, 17, 8), 60 + s) for s in range(3))
    a = oracle.attention_masked(q, k, v, 0.3, False, 16, 16)
    b = oracle.attention_masked(q, k, v, 0.3, False, -1, -1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rows_subset():
    q, k, v = (_rand((2, 2, 25, 8), 70 + s) for s in range(3))
    bias = _rand((1, 2, 25, 25), 74)
    full = oracle.attention_masked(q, k, v, 0.3, True, 7, -1, bias)
    rows = [24, 0, 9]
    sub = oracle.attention_masked(q, k, v, 0.3, True, 7, -1, bias, rows=rows)
    assert np.array_equal(sub[0], full[0][:, :, rows]) and np.array_equal(sub[1], full[1][:, :, rows])


MUTANTS = {
    "bias_scaled": ("sc += bias[b * sb + h * sh + i * si + j];", "sc += scale * bias[b * sb + h * sh + i * si + j];"),
    "bias_transposed": ("sc += bias[b * sb + h * sh + i * si + j];", "sc += bias[b * sb + h * sh + j * si + i];"),
    "head_batch_swapped": ("const int64_t slice = t / R, b = slice / H, h = slice % H;",
                           "const int64_t slice = t / R, h = slice / B, b = slice % B;"),
    "left_window_off_by_one": ("if (wl >= 0 && j < i - wl)", "if (wl >= 0 && j <= i - wl)"),
    "right_window_ignored": ("if (wr >= 0 && j > i + wr)", "if (0)"),
    "empty_row_not_handled": ("if (top == -INFINITY) {", "if (0) {"),
    "causal_ignored": ("if (causal && j > i)", "if (0)"),
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
    lib.oracle_attn_masked_f64.restype = ctypes.c_int
    lib.oracle_attn_masked_f64.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2 + [
        ctypes.c_int64] * 4 + [ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                               ctypes.c_int64, ctypes.c_int]
    return lib


def _passes(lib):
    B, H, N, d = 2, 3, 19, 8
    q, k, v = (np.ascontiguousarray(_rand((B, H, N, d), 80 + s)) for s in range(3))
    cases = [(True, -1, -1, (1, 3)), (False, 4, 2, (2, 1)), (False, -1, -1, (2, 3))]
    for causal, wl, wr, bshape in cases:
        bias = np.broadcast_to(_rand(bshape + (N, N), 85), (B, H, N, N)).copy(order="C")
        bias[1, 2, 5, :] = -np.inf  # one empty row
        o = np.empty((B, H, N, d))
        lse = np.empty((B, H, N))
        lib.oracle_attn_masked_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, bias.ctypes.data, H * N * N, N * N, N,
                                   o.ctypes.data, lse.ctypes.data, B, H, N, d, 0.4, int(causal), wl, wr, None, 0, 1)
        keep = np.ones((B, H, N), dtype=bool)
        keep[1, 2, 5] = False
        o_t, lse_t = _torch_ref(q, k, v, 0.4, causal, wl, wr, bias)
        if not np.isfinite(o).all() or np.abs(o[keep] - o_t[keep]).max() > 1e-12:
            return False
        if np.abs(lse[keep] - lse_t[keep]).max() > 1e-12 or not (np.all(o[1, 2, 5] == 0) and lse[1, 2, 5] == -np.inf):
            return False
    return True


def test_unmodified_source_passes(tmp_path):
    assert _passes(_build(tmp_path, "identity", "int oracle_attn_masked_f64", "int oracle_attn_masked_f64"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    assert not _passes(_build(tmp_path, name, *MUTANTS[name])), name
