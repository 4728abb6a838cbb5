"""The pins must be able to fail: plant plausible mistakes in copies of the
oracle's C source (on the CPU, in a temporary directory), build each mutant and
check that the hand-derived examples or the invariants reject it.
"""
import ctypes
import json
import math
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "attn_oracle.c")

MUTANTS = {
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "scale_twice": ("s[j] = scale * dot;", "s[j] = scale * scale * dot;"),
    "scores_transposed": ("const double *qs = q + (sl * N + i) * d;\n"
                          "            const double *ks = k + sl * N * d;",
                          "const double *qs = k + (sl * N + i) * d;\n"
                          "            const double *ks = q + sl * N * d;"),
    "diagonal_excluded": ("causal ? i + 1 : N", "causal ? (i > 0 ? i : 1) : N"),
    "one_key_leaks": ("causal ? i + 1 : N", "causal ? (i + 2 < N ? i + 2 : N) : N"),
    "no_max_subtraction": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "lse_without_max": ("*lse_out = m + log(sum);", "*lse_out = log(sum);"),
    "not_normalised": ("const double p = s[j] / sum;", "const double p = s[j];"),
    "exp_sign_flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "values_reversed": ("const double *v_row = v + j * d;",
                        "const double *v_row = v + (n_allow - 1 - j) * d;"),
    "dot_misses_last_dim": ("for (int64_t c = 0; c < d; ++c)\n            dot",
                            "for (int64_t c = 0; c + 1 < d; ++c)\n            dot"),
}


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-ffp-contract=off", "-fopenmp",
                    str(path), "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    lib.oracle_attn_f64.restype = ctypes.c_int
    lib.oracle_attn_f64.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 3 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
    return lib


def _run(lib, q, k, v, scale, causal):
    q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
    N, d = q.shape[-2:]
    S = q.size // (N * d)
    o = np.empty_like(q)
    lse = np.empty(q.shape[:-1])
    lib.oracle_attn_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                        lse.ctypes.data, S, N, d, scale, int(causal), None, 0, 1)
    return o, lse


def _pins_pass(lib) -> bool:
    """True when the mutant passes every check (i.e. the mistake went unseen)."""
    with open(os.path.join(HERE, "golden", "hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    with np.errstate(all="ignore"):
        for c in cases:
            for causal in (False, True):
                o, lse = _run(lib, np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                              c["scale"], causal)
                eo = np.array(c["o_causal" if causal else "o"])
                el = np.array(c["lse_causal" if causal else "lse"])
                if not (np.allclose(o, eo, rtol=1e-13, atol=1e-13)
                        and np.allclose(lse, el, rtol=1e-13, atol=1e-13)):
                    return False
        # constant keys: uniform weights, (prefix) mean of values
        r = np.random.default_rng(0)
        N, d = 12, 4
        q = r.standard_normal((N, d))
        k = np.tile(r.standard_normal(d), (N, 1))
        v = r.standard_normal((N, d))
        o, _ = _run(lib, q, k, v, 0.5, True)
        if not np.allclose(o, np.cumsum(v, 0) / np.arange(1, N + 1)[:, None], atol=1e-12):
            return False
    return True


def test_unmodified_oracle_passes_the_same_checks(tmp_path):
    lib = _build(tmp_path, "identity", "s[j] = scale * dot;", "s[j] = scale * dot;")
    assert _pins_pass(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build(tmp_path, name, old, new)
    assert not _pins_pass(lib), f"planted mistake '{name}' passed every pin"
