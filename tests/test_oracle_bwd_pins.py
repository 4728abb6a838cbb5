"""Pins for the fp64 backward oracle, from facts that do not come from its own
derivation:

* central finite differences of the forward oracle (the gradient is, by
  definition, the derivative of the forward function);
* torch.autograd in float64 on the CPU (an independent implementation of the
  chain rule);
* closed forms of the softmax Jacobian: the key gradients sum to zero, the
  value gradients sum to the summed upstream gradient, equal value rows give
  zero query and key gradients, and one key gives dV = dO;
* planted mistakes in copies of the C source must each fail a pin.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "attn_bwd_oracle.c")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _fd_grad(oracle_mod, q, k, v, g, scale, causal, which, h=1e-5):
    """Central finite difference of L = sum(g * O) w.r.t. one input."""
    args = {"q": q, "k": k, "v": v}
    base = args[which]
    grad = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        plus, minus = base.copy(), base.copy()
        plus[idx] += h
        minus[idx] -= h
        a = dict(args, **{which: plus})
        b = dict(args, **{which: minus})
        op, _ = oracle_mod.attention(a["q"], a["k"], a["v"], scale, causal)
        om, _ = oracle_mod.attention(b["q"], b["k"], b["v"], scale, causal)
        grad[idx] = (np.sum(g * op) - np.sum(g * om)) / (2 * h)
    return grad


@pytest.mark.parametrize("causal", [False, True])
def test_matches_finite_differences_of_the_forward(oracle_mod, causal):
    q, k, v, g = (_rand((1, 5, 3), s) for s in range(4))
    scale = 0.8
    dq, dk, dv = oracle_mod.attention_backward(q, k, v, g, scale, causal)
    for name, got in (("q", dq), ("k", dk), ("v", dv)):
        want = _fd_grad(oracle_mod, q, k, v, g, scale, causal, name)
        assert np.abs(got - want).max() <= 1e-8, name


def _torch_grads(q, k, v, g, scale, causal):
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = (q @ k.transpose(-1, -2)) * scale
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ v
    (o * torch.tensor(g)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 17, 8), (3, 64, 16), (1, 1, 4)])
def test_matches_float64_autograd(oracle_mod, causal, shape):
    q, k, v, g = (_rand(shape, 10 + s) for s in range(4))
    scale = 0.3
    got = oracle_mod.attention_backward(q, k, v, g, scale, causal)
    want = _torch_grads(q, k, v, g, scale, causal)
    for a, b in zip(got, want):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_jacobian_closed_forms(oracle_mod, causal):
    q, k, v, g = (_rand((2, 40, 6), 20 + s) for s in range(4))
    dq, dk, dv = oracle_mod.attention_backward(q, k, v, g, 0.5, causal)
    # Each row of dS sums to zero (the softmax is invariant to a shift of
    # its scores), so the key gradients sum to zero.
    assert np.abs(dk.sum(axis=1)).max() <= 1e-12
    # Each row of P sums to one, so the value gradients sum to sum_i dO_i.
    assert np.abs(dv.sum(axis=1) - g.sum(axis=1)).max() <= 1e-12
    # Equal value rows: the output does not depend on the probabilities.
    v_eq = np.broadcast_to(v[:, :1], v.shape).copy()
    dq0, dk0, _ = oracle_mod.attention_backward(q, k, v_eq, g, 0.5, causal)
    assert np.abs(dq0).max() <= 1e-13 and np.abs(dk0).max() <= 1e-13


def test_single_key(oracle_mod):
    q, k, v, g = (_rand((3, 1, 5), 30 + s) for s in range(4))
    dq, dk, dv = oracle_mod.attention_backward(q, k, v, g, 1.3, False)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0
    assert np.abs(dv - g).max() <= 1e-15


def test_causal_first_key_and_last_query(oracle_mod):
    # Causal: the last key is seen only by the last query row; row 0 sees
    # only key 0 (so its query gradient is zero).
    q, k, v, g = (_rand((1, 9, 4), 40 + s) for s in range(4))
    dq, dk, dv = oracle_mod.attention_backward(q, k, v, g, 0.9, True)
    assert np.abs(dq[0, 0]).max() == 0
    # dv of the last key = p_{N-1,N-1} dO_{N-1}
    s = 0.9 * q[0, -1] @ k[0].T
    p = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    assert np.abs(dv[0, -1] - p[-1] * g[0, -1]).max() <= 1e-14


def test_subsets_match_full(oracle_mod):
    q, k, v, g = (_rand((2, 33, 8), 50 + s) for s in range(4))
    full = oracle_mod.attention_backward(q, k, v, g, 0.4, True)
    rows, keys = [0, 5, 32], [31, 2, 17]
    dq, dk, dv = oracle_mod.attention_backward(q, k, v, g, 0.4, True, rows=rows, keys=keys)
    assert np.array_equal(dq, full[0][:, rows])
    assert np.array_equal(dk, full[1][:, keys])
    assert np.array_equal(dv, full[2][:, keys])


# ---------------------------------------------------------------------------
# Planted mistakes must be caught.
# ---------------------------------------------------------------------------
MUTANTS = {
    "dq_scale_dropped": ("                out[c] *= scale;", "                out[c] *= 1.0;"),
    "dk_scale_dropped": ("                    okk[c] *= scale;", "                    okk[c] *= 1.0;"),
    "delta_without_p": ("        D += p * dot(doi, v + j * d, d);", "        D += dot(doi, v + j * d, d);"),
    "ds_sign_flipped": ("                const double ds = p * (dot(doi, v + off + j * d, d) - D[sl * N + i]);",
                        "                const double ds = p * (D[sl * N + i] - dot(doi, v + off + j * d, d));"),
    "dv_wrong_upstream": ("                        ovv[c] += p * doi[c];",
                          "                        ovv[c] += p * (dout + off + j * d)[c];"),
    "dk_uses_keys": ("                        okk[c] += ds * qi[c];", "                        okk[c] += ds * kj[c];"),
    "causal_rows_from_zero": ("            for (int64_t i = causal ? j : 0; i < N; ++i) {",
                              "            for (int64_t i = 0; i < N; ++i) {"),
    "max_not_subtracted": ("        const double p = exp(scale * dot(qi, k + j * d, d) - m) / l;",
                           "        const double p = exp(scale * dot(qi, k + j * d, d)) / l;"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-ffp-contract=off", "-fopenmp", str(path), "-o",
                    str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    lib.oracle_attn_bwd_f64.restype = ctypes.c_int
    lib.oracle_attn_bwd_f64.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 3 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_int]
    return lib


def _run_lib(lib, q, k, v, g, scale, causal):
    q, k, v, g = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, g))
    N, d = q.shape[-2:]
    S = q.size // (N * d)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    rc = lib.oracle_attn_bwd_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data, dq.ctypes.data,
                                 dk.ctypes.data, dv.ctypes.data, S, N, d, scale, int(causal), None, 0, None, 0, 1)
    assert rc == 0
    return dq, dk, dv


def _passes_pins(run):
    for causal in (False, True):
        q, k, v, g = (_rand((2, 12, 5), 60 + s) for s in range(4))
        q = q * 4.0  # large logits: a missing max subtraction matters
        got = run(q, k, v, g, 0.6, causal)
        want = _torch_grads(q, k, v, g, 0.6, causal)
        for a, b in zip(got, want):
            if not np.isfinite(a).all() or np.abs(a - b).max() > 1e-10 * max(1.0, np.abs(b).max()):
                return False
    return True


def test_unmodified_backward_oracle_passes(tmp_path):
    lib = _build_mutant(tmp_path, "identity", "int check_index", "int check_index")
    assert _passes_pins(lambda *a: _run_lib(lib, *a))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_backward_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    assert not _passes_pins(lambda *a: _run_lib(lib, *a)), f"mutant {name} went unnoticed"
