"""GPU parity of the backward (attn_bwd through the C ABI) against the fp64
backward oracle on the same seeded inputs.

Tolerance, per gradient tensor over every checked element: max|dX| <=
BWD_MAX * max|dX_ref| and ||dX||_2 <= BWD_RMS * ||dX_ref||_2.  The kernel's
arithmetic bounds it: the probabilities and dS feed the MFMAs as bf16 (round
to nearest, at most 2^-8 relative each), D = rowsum(dO o O) uses the
bf16-rounded forward output, products accumulate in fp32 and the gradients
are rounded to bf16 (at most 2^-8); the per-element errors are a few 2^-9 to
2^-8 (2-4e-3 each) of the typical gradient magnitude.  Measured on MI355X: normwise 2.0-2.7e-3, max 2-5e-3 of the largest
gradient, so the bounds below keep a margin of about four.  Where the reference gradient vanishes (one key
gives dQ = dK = 0 exactly, while the kernel leaves rounding residue of order
1e-7), the comparison is absolute: denominators are floored at ABS_FLOOR.
"""
import math
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

BWD_MAX, BWD_RMS = 2e-2, 1e-2
ABS_FLOOR = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_124_amd as ea
    ea.load_library()
    return ea


@pytest.fixture(scope="module")
def W():
    from exact_attention_124_amd import workloads
    return workloads


def gpu_grads(ea, q, k, v, g, causal, scale=None):
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, g))
    o, lse = ea.attention(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = ea.attention_backward(qd, kd, vd, o, lse, gd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check(got, ref, what):
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        a = a.double().numpy() if torch.is_tensor(a) else a
        assert np.isfinite(a).all(), f"{what} {name}: non-finite"
        err = np.abs(a - b)
        rmax = err.max() / max(np.abs(b).max(), ABS_FLOOR)
        rrms = np.sqrt((err ** 2).sum() / max((b ** 2).sum(), ABS_FLOOR ** 2 * b.size))
        say(f"  {what} {name}: max|d|/max|ref|={rmax:.2e} rms ratio={rrms:.2e}")
        assert rmax <= BWD_MAX, f"{what} {name}: max relative error {rmax}"
        assert rrms <= BWD_RMS, f"{what} {name}: normwise error {rrms}"


EDGE_N = [1, 17, 64, 100, 257, 1000]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_small_full(ea, W, oracle_mod, d, causal):
    for N in EDGE_N:
        q, k, v = W.make_qkv(1, 2, N, d, torch.bfloat16, seed=200 + N)
        g = W.make_grad(1, 2, N, d, torch.bfloat16, seed=200 + N)
        say(f"[bwd] N={N} d={d} causal={causal}")
        ref = oracle_mod.attention_backward(q, k, v, g, 1 / math.sqrt(d), causal)
        check(gpu_grads(ea, q, k, v, g, causal), ref, f"N={N}")


def test_backward_gpt2_heads_full(ea, W, oracle_mod):
    w = W.WORKLOADS["gpt2_heads_bf16"]
    say(f"[bwd] {w.describe()}")
    q, k, v = W.workload_inputs(w)
    g = W.make_grad(w.B, w.H, w.N, w.d, w.dtype, w.seed)
    ref = oracle_mod.attention_backward(q, k, v, g, w.scale, w.causal)
    check(gpu_grads(ea, q, k, v, g, w.causal), ref, "gpt2 heads")


@pytest.mark.parametrize("name,nslices,nsamp", [("causal_2k_bf16", 2, 64), ("dense_8k_bf16", 1, 32),
                                                 ("causal_32k_qx8_bf16", 1, 16)])
def test_backward_sampled(ea, W, oracle_mod, name, nslices, nsamp):
    w = W.WORKLOADS[name]
    say(f"[bwd] {w.describe()} (sampled rows and keys)")
    q, k, v = W.workload_inputs(w)
    g = W.make_grad(w.B, w.H, w.N, w.d, w.dtype, w.seed)
    dq, dk, dv = gpu_grads(ea, q, k, v, g, w.causal)
    slices = W.check_slices(w)[:nslices]
    rows = W.sample_rows(w.N, nsamp, seed=4)
    keys = W.sample_rows(w.N, nsamp, seed=5)
    flat = lambda t: t.reshape(-1, w.N, w.d)[slices]  # noqa: E731
    ref = oracle_mod.attention_backward(flat(q), flat(k), flat(v), flat(g), w.scale, w.causal,
                                        rows=rows, keys=keys)
    got = (flat(dq)[:, rows], flat(dk)[:, keys], flat(dv)[:, keys])
    check(got, ref, name)


def test_backward_causal_paired_odd_block_count(ea, W, oracle_mod):
    # B*H*ceil(N/128) >= 1024 pairs the causal key blocks (dK, dV) and query
    # blocks (dQ); N = 17 * 128 leaves one workgroup per slice with the middle
    # block alone.  Rows and keys are taken from the first, middle and last
    # blocks and from block boundaries.
    B, H, N, d = 1, 64, 17 * 128, 128
    q, k, v = W.make_qkv(B, H, N, d, torch.bfloat16, seed=91)
    g = W.make_grad(B, H, N, d, torch.bfloat16, seed=91)
    say(f"[bwd] causal B={B} H={H} N={N} (17 blocks of 128)")
    dq, dk, dv = gpu_grads(ea, q, k, v, g, True)
    idx = [0, 1, 127, 128, 1023, 1024, 1100, 1151, 1152, 2047, 2048, N - 1]
    slices = [0, B * H - 1]
    flat = lambda t: t.reshape(-1, N, d)[slices]  # noqa: E731
    ref = oracle_mod.attention_backward(flat(q), flat(k), flat(v), flat(g), 1 / math.sqrt(d), True,
                                        rows=idx, keys=idx)
    check((flat(dq)[:, idx], flat(dk)[:, idx], flat(dv)[:, idx]), ref, "paired, 17 blocks")


@pytest.mark.parametrize("d,N", [(128, 1500), (64, 2100)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_ragged_multiblock(ea, W, oracle_mod, d, N, causal):
    # Several key and query blocks with a ragged end: the dK/dV kernel's
    # masked diagonal and tail tiles, its statistics block past N (zeros), and
    # the dQ kernel's separate interior and edge loops.  Rows and keys at block
    # and tile boundaries plus a seeded sample, in every slice.
    B, H = 2, 3
    q, k, v = W.make_qkv(B, H, N, d, torch.bfloat16, seed=300 + N)
    g = W.make_grad(B, H, N, d, torch.bfloat16, seed=300 + N)
    say(f"[bwd] ragged B={B} H={H} N={N} d={d} causal={causal}")
    dq, dk, dv = gpu_grads(ea, q, k, v, g, causal)
    edges = [0, 31, 32, 63, 64, 127, 128, 255, 256, N // 2, N - 65, N - 64, N - 33, N - 32, N - 2, N - 1]
    idx = sorted(set(i for i in edges if 0 <= i < N) | set(W.sample_rows(N, 24, seed=6)))
    flat = lambda t: t.reshape(-1, N, d)  # noqa: E731
    ref = oracle_mod.attention_backward(flat(q), flat(k), flat(v), flat(g), 1 / math.sqrt(d), causal,
                                        rows=idx, keys=idx)
    check((flat(dq)[:, idx], flat(dk)[:, idx], flat(dv)[:, idx]), ref, f"ragged N={N} d={d}")


def test_backward_closed_forms_and_determinism(ea, W):
    q, k, v = (t.cuda() for t in W.make_qkv(2, 4, 700, 128, torch.bfloat16, seed=31))
    g = W.make_grad(2, 4, 700, 128, torch.bfloat16, seed=31).cuda()
    for causal in (False, True):
        o, lse = ea.attention(q, k, v, causal=causal)
        a = ea.attention_backward(q, k, v, o, lse, g, causal=causal)
        b = ea.attention_backward(q, k, v, o, lse, g, causal=causal)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), "backward is not deterministic"
        dq, dk, dv = (t.float() for t in a)
        # Key gradients sum to zero; value gradients sum to the summed dO.
        s_dk = dk.sum(dim=2).abs().max().item()
        s_dv = (dv.sum(dim=2) - g.float().sum(dim=2)).abs().max().item()
        say(f"  causal={causal}: max|sum_j dK_j|={s_dk:.3e}  max|sum dV - sum dO|={s_dv:.3e}")
        assert s_dk <= 2e-2 * dk.abs().max().item() * math.sqrt(700)
        assert s_dv <= 2e-2 * g.float().sum(dim=2).abs().max().item() + 0.1


def test_backward_rejects_missing_workspace(ea):
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 1, 64, dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    with pytest.raises(ea.AttnError) as ei:
        ea.attn_bwd(q, q.clone(), q.clone(), q.clone(), lse, q.clone(), dq, dk, dv, ws)
    assert ei.value.status == ea.STATUS["ATTN_ERR_WORKSPACE"]
