"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself (hand-derived closed forms, invariants of the definition,
special cases that reduce to a textbook identity, and an independent library
computation).  CPU only.

The definition pinned is the one in the grasp.study lesson on standard
self-attention, section "The Computational Steps of Standard Self-Attention":
scores = Q K^T (times the scale), row-wise softmax, output = P V.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))

with open(os.path.join(HERE, "golden", "hand_examples.json")) as f:
    GOLDEN = json.load(f)["cases"]


def rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("case", GOLDEN, ids=[c["name"] for c in GOLDEN])
@pytest.mark.parametrize("causal", [False, True])
def test_hand_derived_examples(oracle_mod, case, causal):
    q = np.array(case["q"], dtype=np.float64)
    k = np.array(case["k"], dtype=np.float64)
    v = np.array(case["v"], dtype=np.float64)
    o, lse = oracle_mod.attention(q, k, v, case["scale"], causal=causal)
    exp_o = np.array(case["o_causal" if causal else "o"])
    exp_l = np.array(case["lse_causal" if causal else "lse"])
    np.testing.assert_allclose(o, exp_o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, exp_l, rtol=1e-13, atol=1e-13)


def test_single_key_returns_value_row(oracle_mod):
    # N = 1: the softmax of one score is 1, so o = v and lse = the score.
    r = rng(0)
    for d in (1, 7, 64, 128):
        q, k, v = (r.standard_normal((3, 1, d)) for _ in range(3))
        o, lse = oracle_mod.attention(q, k, v, 0.3, causal=False)
        np.testing.assert_array_equal(o, v)
        np.testing.assert_allclose(lse[:, 0], 0.3 * np.einsum("sc,sc->s", q[:, 0], k[:, 0]),
                                   rtol=1e-14, atol=1e-14)


def test_identity_values_expose_probabilities(oracle_mod):
    # With V = I (d = N) the output is P itself: rows are non-negative and sum to 1,
    # and each row equals exp(s - lse) with s the scaled scores.
    r = rng(1)
    N = 9
    q = r.standard_normal((2, N, N))
    k = r.standard_normal((2, N, N))
    v = np.broadcast_to(np.eye(N), (2, N, N)).copy()
    for causal in (False, True):
        P, lse = oracle_mod.attention(q, k, v, 0.5, causal=causal)
        assert (P >= 0).all()
        np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-14)
        s = 0.5 * np.einsum("sic,sjc->sij", q, k)
        expect = np.exp(s - lse[..., None])
        if causal:
            expect = np.tril(expect)
            assert np.all(np.triu(P, 1) == 0.0)
        np.testing.assert_allclose(P, expect, rtol=1e-12, atol=1e-15)


def test_ones_values_give_ones(oracle_mod):
    r = rng(2)
    q, k = r.standard_normal((2, 4, 33, 16))
    v = np.ones((4, 33, 16))
    for causal in (False, True):
        o, _ = oracle_mod.attention(q, k, v, 0.25, causal=causal)
        np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


def test_constant_keys_average_values(oracle_mod):
    # Every key equal to k0: the scores of a row are all equal, P is uniform over the
    # allowed keys, o is the (prefix) mean of V, lse = scale*q.k0 + ln(count).
    r = rng(3)
    N, d, scale = 40, 8, 0.7
    q = r.standard_normal((N, d))
    k0 = r.standard_normal(d)
    k = np.tile(k0, (N, 1))
    v = r.standard_normal((N, d))
    o, lse = oracle_mod.attention(q, k, v, scale, causal=False)
    np.testing.assert_allclose(o, np.tile(v.mean(0), (N, 1)), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, scale * q @ k0 + math.log(N), rtol=1e-13, atol=1e-13)
    o, lse = oracle_mod.attention(q, k, v, scale, causal=True)
    prefix = np.cumsum(v, 0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(o, prefix, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, scale * q @ k0 + np.log(np.arange(1, N + 1)),
                               rtol=1e-13, atol=1e-13)


def test_key_permutation_invariance_and_query_equivariance(oracle_mod):
    r = rng(4)
    N, d = 50, 16
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    o, lse = oracle_mod.attention(q, k, v, 0.25)
    pk = r.permutation(N)
    o2, lse2 = oracle_mod.attention(q, k[pk], v[pk], 0.25)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)
    pq = r.permutation(N)
    o3, lse3 = oracle_mod.attention(q[pq], k, v, 0.25)
    np.testing.assert_allclose(o3, o[pq], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse3, lse[pq], rtol=1e-13, atol=1e-13)


def test_key_shift_moves_lse_only(oracle_mod):
    # k_j <- k_j + u adds scale*q_i.u to every score of row i: P unchanged, lse shifted.
    r = rng(5)
    N, d, scale = 30, 8, 0.4
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    u = r.standard_normal(d)
    for causal in (False, True):
        o, lse = oracle_mod.attention(q, k, v, scale, causal=causal)
        o2, lse2 = oracle_mod.attention(q, k + u, v, scale, causal=causal)
        np.testing.assert_allclose(o2, o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse2, lse + scale * q @ u, rtol=1e-12, atol=1e-12)


def test_linear_in_values(oracle_mod):
    r = rng(6)
    N, d = 25, 12
    q, k, v1, v2 = (r.standard_normal((N, d)) for _ in range(4))
    for causal in (False, True):
        o1, _ = oracle_mod.attention(q, k, v1, 0.3, causal=causal)
        o2, _ = oracle_mod.attention(q, k, v2, 0.3, causal=causal)
        o3, _ = oracle_mod.attention(q, k, 2.5 * v1 - 0.5 * v2, 0.3, causal=causal)
        np.testing.assert_allclose(o3, 2.5 * o1 - 0.5 * o2, rtol=1e-11, atol=1e-12)


def test_output_in_convex_hull_of_allowed_values(oracle_mod):
    r = rng(7)
    N, d = 40, 6
    q, k, v = (3 * r.standard_normal((N, d)) for _ in range(3))
    o, _ = oracle_mod.attention(q, k, v, 1.0, causal=True)
    for i in range(N):
        lo = v[: i + 1].min(0)
        hi = v[: i + 1].max(0)
        assert np.all(o[i] >= lo - 1e-12) and np.all(o[i] <= hi + 1e-12)


def test_causal_row_equals_unmasked_attention_on_its_prefix(oracle_mod):
    # Row i of causal attention is plain attention of query i over keys 0..i; this pins
    # that the diagonal is included and nothing after it leaks in.
    r = rng(8)
    N, d = 24, 8
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    o, lse = oracle_mod.attention(q, k, v, 0.35, causal=True)
    for i in range(N):
        oi, li = oracle_mod.attention(np.tile(q[i], (i + 1, 1)), k[: i + 1], v[: i + 1], 0.35)
        np.testing.assert_allclose(o[i], oi[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[i], li[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(o[0], v[0])
    np.testing.assert_allclose(lse[0], 0.35 * q[0] @ k[0], rtol=1e-14)


def test_scale_acts_on_scores(oracle_mod):
    # softmax(scale * q.k) depends on q and scale only through scale*q.
    r = rng(9)
    N, d = 20, 8
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    o1, l1 = oracle_mod.attention(q, k, v, 0.125)
    o2, l2 = oracle_mod.attention(0.125 * q, k, v, 1.0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)


def test_matches_independent_float64_library_computation(oracle_mod):
    # torch's float64 CPU softmax and matmul: code that shares nothing with the C oracle.
    g = torch.Generator().manual_seed(10)
    for (S, N, d, causal) in [(3, 17, 64, False), (2, 65, 128, True), (1, 128, 64, False),
                              (4, 31, 5, True)]:
        q, k, v = (torch.randn(S, N, d, generator=g, dtype=torch.float64) for _ in range(3))
        scale = 1 / math.sqrt(d)
        s = (q @ k.transpose(-1, -2)) * scale
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        ref_o = torch.softmax(s, -1) @ v
        ref_l = torch.logsumexp(s, -1)
        o, lse = oracle_mod.attention(q, k, v, scale, causal=causal)
        np.testing.assert_allclose(o, ref_o.numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, ref_l.numpy(), rtol=1e-12, atol=1e-12)


def test_row_subset_matches_full(oracle_mod):
    r = rng(11)
    q, k, v = (r.standard_normal((3, 70, 16)) for _ in range(3))
    rows = [0, 5, 69, 33]
    for causal in (False, True):
        o, lse = oracle_mod.attention(q, k, v, 0.2, causal=causal)
        os_, ls_ = oracle_mod.attention(q, k, v, 0.2, causal=causal, rows=rows)
        np.testing.assert_array_equal(os_, o[:, rows])
        np.testing.assert_array_equal(ls_, lse[:, rows])


def test_thread_count_does_not_change_bits(oracle_mod):
    r = rng(12)
    q, k, v = (r.standard_normal((4, 64, 32)) for _ in range(3))
    a = oracle_mod.attention(q, k, v, 0.2, causal=True, threads=1)
    b = oracle_mod.attention(q, k, v, 0.2, causal=True, threads=8)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_rejects_bad_rows(oracle_mod):
    q = np.zeros((1, 4, 2))
    with pytest.raises(RuntimeError):
        oracle_mod.attention(q, q, q, 1.0, rows=[4])
    with pytest.raises(RuntimeError):
        oracle_mod.attention(q, q, q, 1.0, rows=[-1])


def test_bf16_inputs_upcast_exactly(oracle_mod):
    # bf16 -> fp64 is exact, so the oracle sees exactly the values the device sees.
    g = torch.Generator().manual_seed(13)
    q, k, v = (torch.randn(1, 2, 16, 64, generator=g).to(torch.bfloat16) for _ in range(3))
    o1, l1 = oracle_mod.attention(q, k, v, 0.125)
    o2, l2 = oracle_mod.attention(q.float().numpy().astype(np.float64), k.float().numpy(),
                                  v.float().numpy(), 0.125)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
