"""GPU parity of the fp8 fused forward (OCP E4M3 inputs, and E5M2 or mixed
formats through attn_fwd_fp8_fmt) against the fp64 oracle on the
dequantised inputs.

Tolerance, derived from the kernel's arithmetic.  Both sides see the same
inputs exactly (an E4M3 code times an fp32 factor), and the scores, softmax
and accumulations are fp32.  What differs: the kernel rounds each
probability P (taken relative to a reference maximum that is one of the
row's own scores, so the row sum l >= 1) to E4M3 before the second product,
while the normaliser l sums the unrounded values, and it rounds O to bf16.
E4M3 rounding moves P by at most 2^-4 P in the normal range (P >= 2^-6) and
by at most min(P, 2^-10) below it (subnormal step 2^-9).  Dividing by l >= 1,
with p = P / l the exact weights,

    |dO_ic| <= 2^-4 A_ic + B_ic + bf16 and fp32 terms,
    A_ic = sum_j p_ij |V_jc|,   B_ic = sum_j min(p_ij, 2^-10) |V_jc|,

which the tests check element by element as

    |dO_ic| <= (2^-4 + 2^-10) A_ic + B_ic + 2^-8 |O_ic| + 1e-6

(2^-8 |O| is the bf16 rounding of O, an 8-bit significand; the extra
2^-10 A absorbs fp32 accumulation).
The weights p come from the oracle.  lse comes from fp32 scores and sums:
|dlse| <= 1e-3 as for the bf16 kernel.
"""
import math
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-3


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


def check(oracle_mod, o, lse, q8, k8, v8, qd, kd, vd, scale, causal, what, rows=None):
    ro, rl = oracle_mod.attention_fp8(q8, k8, v8, qd, kd, vd, scale, causal, rows=rows)
    w = oracle_mod.probabilities(oracle_mod.dequantize_fp8(q8, qd), oracle_mod.dequantize_fp8(k8, kd), scale,
                                 causal, rows=rows)
    va = np.abs(oracle_mod.dequantize_fp8(v8, vd))
    a = w @ va
    b = np.minimum(w, 2.0 ** -10) @ va
    o = o.double().cpu().numpy().reshape(ro.shape)
    lse = lse.double().cpu().numpy().reshape(rl.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - ro)
    bound = (2.0 ** -4 + 2.0 ** -10) * a + b + 2.0 ** -8 * np.abs(ro) + 1e-6
    ratio = (err / bound).max()
    lerr = np.abs(lse - rl).max()
    say(f"  {what}: max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} max err/bound={ratio:.3f} "
        f"max|dlse|={lerr:.3e}")
    assert ratio <= 1.0, f"{what}: error above the E4M3 rounding bound (ratio {ratio})"
    assert lerr <= LSE_TOL, f"{what}: lse error {lerr}"


def run(ea, q8, k8, v8, qd, kd, vd, causal, scale=None):
    o, lse = ea.attention_fp8(q8.cuda(), k8.cuda(), v8.cuda(), qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 64, 100, 257, 1000])
def test_small_full(ea, W, oracle_mod, N, d, causal):
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(1, 2, N, d, seed=N + d, q_mult=2.0)
    scale = 1 / math.sqrt(d)
    say(f"[fp8] B=1 H=2 N={N} d={d} causal={causal}")
    o, lse = run(ea, q8, k8, v8, qd, kd, vd, causal)
    check(oracle_mod, o, lse, q8, k8, v8, qd, kd, vd, scale, causal, f"N={N} d={d} causal={causal}")


def test_gpt2_heads_full(ea, W, oracle_mod):
    say("[fp8] non-causal B=1 H=12 N=1024 d=64")
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(1, 12, 1024, 64, seed=0)
    o, lse = run(ea, q8, k8, v8, qd, kd, vd, False)
    check(oracle_mod, o, lse, q8, k8, v8, qd, kd, vd, 1 / 8, False, "gpt2 heads")


def _sliced(ea, W, oracle_mod, B, H, N, d, causal, q_mult, n_slices, n_rows, label, formats=("e4m3",) * 3):
    say(f"[fp8] {label} B={B} H={H} N={N} d={d} causal={causal} q_mult={q_mult} formats={formats} (sampled)")
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(B, H, N, d, seed=0, q_mult=q_mult, formats=formats)
    o, lse = run(ea, q8, k8, v8, qd, kd, vd, causal)
    g = torch.Generator().manual_seed(1)
    slices = torch.randperm(B * H, generator=g)[:n_slices].tolist()
    rows = W.sample_rows(N, n_rows, seed=2) if n_rows < N else None
    def pick(t):
        return t.reshape(B * H, N, -1)[slices]
    r = torch.tensor(rows) if rows is not None else torch.arange(N)
    check(oracle_mod, o.reshape(B * H, N, d)[slices][:, r], lse.reshape(B * H, N)[slices][:, r],
          pick(q8), pick(k8), pick(v8), qd, kd, vd, 1 / math.sqrt(d), causal, label, rows=rows)


def test_causal_2k(ea, W, oracle_mod):
    _sliced(ea, W, oracle_mod, 4, 32, 2048, 128, True, 1.0, 2, 2048, "causal 2k")


def test_dense_8k(ea, W, oracle_mod):
    _sliced(ea, W, oracle_mod, 8, 32, 8192, 128, False, 1.0, 2, 64, "dense 8k")


def test_causal_paired_odd_block_count(ea, W, oracle_mod):
    # B*H*ceil(N/128) >= 1024 pairs causal query blocks; N = 17 * 128 leaves
    # one workgroup per slice with the middle block alone.  All rows checked.
    _sliced(ea, W, oracle_mod, 1, 64, 17 * 128, 128, True, 1.0, 2, 17 * 128, "causal paired, 17 blocks")


def test_causal_32k_qx8(ea, W, oracle_mod):
    _sliced(ea, W, oracle_mod, 1, 32, 32768, 128, True, 8.0, 2, 32, "causal 32k Qx8")


def test_v_descale_is_a_pure_output_factor(ea, W):
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(2, 4, 300, 128, seed=9)
    o1, l1 = run(ea, q8, k8, v8, qd, kd, vd, True)
    o2, l2 = run(ea, q8, k8, v8, qd, kd, 2 * vd, True)
    assert torch.equal(o2.float(), 2 * o1.float()) and torch.equal(l1, l2)


def test_deterministic(ea, W):
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(2, 16, 2048, 128, seed=5)
    a = run(ea, q8, k8, v8, qd, kd, vd, False)
    b = run(ea, q8, k8, v8, qd, kd, vd, False)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_rejects_bad_descale_and_dtype(ea, W):
    q8, k8, v8, qd, kd, vd = (t.cuda() if torch.is_tensor(t) else t for t in W.make_qkv_fp8(1, 1, 64, 64))
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(ea.AttnError):
            ea.attention_fp8(q8, k8, v8, qd, bad, vd)
    with pytest.raises(TypeError):
        ea.attention_fp8(q8.view(torch.uint8), k8, v8, qd, kd, vd)


# ---------------------------------------------------------------------------
# Inputs in OCP E5M2, alone or mixed with E4M3 (attn_fwd_fp8_fmt).  Both
# sides read the same codes exactly and the kernel still rounds P to E4M3, so
# the bound above holds unchanged.
# ---------------------------------------------------------------------------
ALL_FORMATS = [(a, b, c) for a in ("e4m3", "e5m2") for b in ("e4m3", "e5m2") for c in ("e4m3", "e5m2")]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("formats", ALL_FORMATS)
def test_formats_small(ea, W, oracle_mod, formats, d, causal):
    N = 257
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(1, 2, N, d, seed=11 + d, q_mult=2.0, formats=formats)
    say(f"[fp8] formats={formats} B=1 H=2 N={N} d={d} causal={causal}")
    o, lse = run(ea, q8, k8, v8, qd, kd, vd, causal)
    check(oracle_mod, o, lse, q8, k8, v8, qd, kd, vd, 1 / math.sqrt(d), causal, f"{formats} d={d} causal={causal}")


@pytest.mark.parametrize("N", [1, 17, 1000])
def test_e5m2_ragged(ea, W, oracle_mod, N):
    f = ("e5m2",) * 3
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(2, 3, N, 64, seed=N, q_mult=4.0, formats=f)
    say(f"[fp8] e5m2 B=2 H=3 N={N} d=64 causal")
    o, lse = run(ea, q8, k8, v8, qd, kd, vd, True)
    check(oracle_mod, o, lse, q8, k8, v8, qd, kd, vd, 1 / 8, True, f"e5m2 N={N}")


def test_dense_8k_e5m2(ea, W, oracle_mod):
    _sliced(ea, W, oracle_mod, 8, 32, 8192, 128, False, 1.0, 2, 64, "dense 8k e5m2", formats=("e5m2",) * 3)


def test_causal_2k_e5m2_values(ea, W, oracle_mod):
    _sliced(ea, W, oracle_mod, 4, 32, 2048, 128, True, 1.0, 2, 2048, "causal 2k, e5m2 V",
            formats=("e4m3", "e4m3", "e5m2"))


def test_fmt_entry_reads_bytes_in_the_given_formats(ea, W, oracle_mod):
    f = ("e5m2", "e4m3", "e5m2")
    q8, k8, v8, qd, kd, vd = (t.cuda() if torch.is_tensor(t) else t
                              for t in W.make_qkv_fp8(1, 4, 300, 128, seed=12, formats=f))
    say("[fp8] attn_fwd_fp8_fmt on raw bytes, B=1 H=4 N=300 d=128")
    o1, l1 = ea.attention_fp8(q8, k8, v8, qd, kd, vd, causal=True)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    F = ea.FP8_FORMATS
    u8 = [t.view(torch.uint8) for t in (q8, k8, v8)]
    ea.attn_fwd_fp8_fmt(*u8, o2, l2, qd, kd, vd, F["e5m2"], F["e4m3"], F["e5m2"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # The same bytes read as all-E4M3 are another input, and the kernel
    # follows that reading: it matches the oracle for it.
    o3, l3 = torch.empty_like(o1), torch.empty_like(l1)
    ea.attn_fwd_fp8_fmt(*u8, o3, l3, qd, kd, vd, 0, 0, 0, causal=True)
    torch.cuda.synchronize()
    assert not torch.equal(o3, o1)
    cpu = [t.cpu() for t in u8]  # uint8: the oracle reads these as E4M3
    check(oracle_mod, o3.cpu(), l3.cpu(), *cpu, qd, kd, vd, 1 / math.sqrt(128), True, "bytes read as e4m3")
    with pytest.raises(ea.AttnError):
        ea.attn_fwd_fp8_fmt(*u8, o3, l3, qd, kd, vd, 2, 0, 0)
