"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Tolerances (bf16 inputs, unit-variance data): over every checked element,
max|dO| <= 2e-2 and mean|dO| <= 2e-3.  fp32 path: max|dO| <= 1e-5 * max|O_ref|
(normwise; an element-wise relative bound is ill-posed where O ~ 0).  lse:
the fused bf16 kernel's row sum adds the probabilities as rounded to bf16 for
P*V, each within 2^-8 of its fp32 value, so ln(sum) moves by at most
ln(1 + 2^-8) = 3.9e-3 (scores and sums are fp32, adding well under 1e-4):
|dlse| <= 4e-3; fp32 |dlse| <= 1e-5 * max(1, |lse|); unfused bf16 scores are
rounded to bf16 before the softmax (whose sum is fp32), so its lse may move by
up to 2^-8 of the largest |scaled score| (bounded by scale * max|q| * max|k|)
plus 1e-3.
"""
import math
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, BF16_LSE = 2e-2, 2e-3, 4e-3
UNFUSED_LSE_BASE = 1e-3
F32_REL = 1e-5


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


def check_bf16(o, lse, ro, rl, what, lse_tol=BF16_LSE):
    o = o.double().cpu().numpy() if torch.is_tensor(o) else o
    lse = lse.double().cpu().numpy() if torch.is_tensor(lse) else lse
    err = np.abs(o - ro)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    mx, mean = err.max(), err.mean()
    lerr = np.abs(lse - rl).max()
    say(f"  {what}: max|dO|={mx:.3e} mean|dO|={mean:.3e} max|dlse|={lerr:.3e}")
    assert mx <= BF16_MAX, f"{what}: max abs error {mx}"
    assert mean <= BF16_MEAN, f"{what}: mean abs error {mean}"
    assert lerr <= lse_tol, f"{what}: lse error {lerr}"


def check_f32(o, lse, ro, rl, what):
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    assert np.isfinite(o).all()
    mx = np.abs(o - ro).max()
    ref = np.abs(ro).max()
    lerr = (np.abs(lse - rl) / np.maximum(1.0, np.abs(rl))).max()
    say(f"  {what}: max|dO|/max|O|={mx / ref:.3e} max rel dlse={lerr:.3e}")
    assert mx <= F32_REL * ref, f"{what}: normwise error {mx / ref}"
    assert lerr <= F32_REL, f"{what}: lse error {lerr}"


def unfused_lse_tol(q, k, scale):
    qn = q.float().norm(dim=-1).max().item()
    kn = k.float().norm(dim=-1).max().item()
    return 2.0 ** -8 * scale * qn * kn + UNFUSED_LSE_BASE


def run(ea, q, k, v, causal, scale=None, variant="fused"):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    if variant == "fused":
        o, lse = ea.attention(qd, kd, vd, causal=causal, scale=scale)
    else:
        o, lse, ws = ea.attention_unfused(qd, kd, vd, causal=causal, scale=scale)
        del ws
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------
def test_small_fp32_full(ea, W, oracle_mod):
    w = W.WORKLOADS["small_fp32"]
    say(f"[parity] {w.describe()}")
    q, k, v = W.workload_inputs(w)
    ro, rl = oracle_mod.attention(q, k, v, w.scale, w.causal)
    o, lse = run(ea, q, k, v, w.causal)
    check_f32(o, lse, ro, rl, "fused fp32")
    o, lse = run(ea, q, k, v, w.causal, variant="unfused")
    check_f32(o, lse, ro, rl, "unfused fp32")


def test_gpt2_heads_bf16_full(ea, W, oracle_mod):
    w = W.WORKLOADS["gpt2_heads_bf16"]
    say(f"[parity] {w.describe()}")
    q, k, v = W.workload_inputs(w)
    ro, rl = oracle_mod.attention(q, k, v, w.scale, w.causal)
    o, lse = run(ea, q, k, v, w.causal)
    check_bf16(o, lse, ro, rl, "fused bf16")
    o, lse = run(ea, q, k, v, w.causal, variant="unfused")
    check_bf16(o, lse, ro, rl, "unfused bf16", unfused_lse_tol(q, k, w.scale))


def _named_slices(ea, W, oracle_mod, name, extra_rows, variants=("fused",)):
    # Every row of the slices the workload names for the oracle (all slices
    # when it names none) is compared element by element; a few seeded rows
    # of every other slice are checked as well.
    w = W.WORKLOADS[name]
    slices = W.check_slices(w)
    say(f"[parity] {w.describe()}: every row of {len(slices)} slices")
    q, k, v = W.workload_inputs(w)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    qs = q.reshape(-1, w.N, w.d)[slices]
    ks = k.reshape(-1, w.N, w.d)[slices]
    vs = v.reshape(-1, w.N, w.d)[slices]
    ro, rl = oracle_mod.attention(qs, ks, vs, w.scale, w.causal)
    say(f"  oracle done on {len(slices)} full slices")
    all_rows = W.sample_rows(w.N, extra_rows, seed=3)
    ro2, rl2 = oracle_mod.attention(q.reshape(-1, w.N, w.d), k.reshape(-1, w.N, w.d),
                                    v.reshape(-1, w.N, w.d), w.scale, w.causal, rows=all_rows)
    del qs, ks, vs
    for variant in variants:
        if variant == "fused":
            o, lse = ea.attention(qd, kd, vd, causal=w.causal)
            tol = BF16_LSE
        else:
            o, lse, ws = ea.attention_unfused(qd, kd, vd, causal=w.causal)
            del ws
            tol = unfused_lse_tol(q, k, w.scale)
        torch.cuda.synchronize()
        of = o.reshape(-1, w.N, w.d)
        lf = lse.reshape(-1, w.N)
        sl = torch.tensor(slices, device=o.device)
        check_bf16(of[sl], lf[sl], ro, rl, f"{variant} {len(slices)} slices x all {w.N} rows", tol)
        arw = torch.tensor(all_rows, device=o.device)
        check_bf16(of[:, arw], lf[:, arw], ro2, rl2,
                   f"{variant} all {of.shape[0]} slices x {len(all_rows)} rows", tol)
        assert torch.isfinite(o).all().item(), "non-finite output somewhere"
        del o, lse, of, lf
        torch.cuda.empty_cache()
    del qd, kd, vd
    torch.cuda.empty_cache()


def test_causal_2k_bf16_every_slice(ea, W, oracle_mod):
    _named_slices(ea, W, oracle_mod, "causal_2k_bf16", 8, variants=("fused", "unfused"))


def test_dense_8k_bf16_named_slices(ea, W, oracle_mod):
    _named_slices(ea, W, oracle_mod, "dense_8k_bf16", 6, variants=("fused", "unfused"))


def test_causal_32k_qx8_bf16_named_heads(ea, W, oracle_mod):
    # The unfused path is not parity-gated here: its bf16 scores carry absolute
    # errors of ~0.25 at logits near 32, beyond the 2e-2 output bound.
    _named_slices(ea, W, oracle_mod, "causal_32k_qx8_bf16", 4)


def test_causal_odd_block_count_eight_waves(ea, W, oracle_mod):
    # B*H*ceil(N/256) >= 1024 and N > 4096 select the 8-wave causal kernel; with
    # N = 17 * 256 one workgroup of each slice runs the middle query block alone
    # and the others run blocks 16-i and i.  Rows are taken from the first,
    # middle and last blocks and from block boundaries.
    B, H, N, d = 1, 64, 17 * 256, 128
    q, k, v = W.make_qkv(B, H, N, d, torch.bfloat16, seed=77)
    rows = [0, 1, 255, 256, 2047, 2048, 2049, 2200, 2303, 2304, 4095, 4096, 4200, N - 1]
    slices = [0, 31, B * H - 1]
    say(f"[parity] causal B={B} H={H} N={N} (17 query blocks of 256), rows {rows}")
    qs, ks, vs = (t.reshape(-1, N, d)[slices] for t in (q, k, v))
    ro, rl = oracle_mod.attention(qs, ks, vs, 1 / math.sqrt(d), True, rows=rows)
    o, lse = ea.attention(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    sl, rw = torch.tensor(slices, device=o.device), torch.tensor(rows, device=o.device)
    check_bf16(o.reshape(-1, N, d)[sl][:, rw], lse.reshape(-1, N)[sl][:, rw], ro, rl, "fused, odd block count")
    assert torch.isfinite(o).all().item()


@pytest.mark.parametrize("N", [4100, 2049])
def test_wide_split_ragged(ea, W, oracle_mod, N):
    # Non-causal d = 64 on a small grid with long key walks (one slice; 16 or
    # more 32-key tiles per wave at four waves) runs the split-key kernel with
    # 8 waves x 64 rows: every K and V operand feeds two 32-row blocks and
    # eight partial states are merged.  Ragged N ends in a partial tile and a
    # partial 64-row block.  Every row is checked.
    B, H, d = 1, 1, 64
    q, k, v = W.make_qkv(B, H, N, d, torch.bfloat16, seed=40 + N)
    say(f"[parity] wide split-key B={B} H={H} N={N} d={d}")
    ro, rl = oracle_mod.attention(q, k, v, 1 / math.sqrt(d), False)
    o, lse = run(ea, q, k, v, False)
    check_bf16(o, lse, ro, rl, "fused, 8-wave split-key")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_eight_wave_ragged(ea, W, oracle_mod, d, causal):
    # Grids of at least 192 256-row blocks (and, causal, N > 1024) select the
    # 8-wave K-ahead kernels; N = 1000 and 4100 end in a partial 64-key tile,
    # so the last steps take the checked path (masked tail keys, and for
    # causal the diagonal), after the unchecked main loop.  Rows come from
    # the first block, tile and block boundaries and the ragged end.
    N = 4100 if causal else 1000
    B, H = (1, 64) if causal else (4, 64)
    _eight_wave_case(ea, W, oracle_mod, B, H, N, d, causal)


@pytest.mark.parametrize("d", [64, 128])
def test_eight_wave_causal_unpaired_mid_length(ea, W, oracle_mod, d):
    # Causal N = 1500 on 64 slices: 6 blocks of 256 rows per slice, 384
    # workgroups (at least 192 and N > 1024: the 8-wave kernel; fewer than two
    # rounds: unpaired, longest block first), ragged last tile and block.
    _eight_wave_case(ea, W, oracle_mod, 1, 64, 1500, d, True)


def _eight_wave_case(ea, W, oracle_mod, B, H, N, d, causal):
    q, k, v = W.make_qkv(B, H, N, d, torch.bfloat16, seed=900 + d + causal)
    rows = sorted({0, 1, 63, 64, 255, 256, N // 2, N - 66, N - 65, N - 64, N - 5, N - 1})
    slices = [0, 37, B * H - 1]
    say(f"[parity] 8-wave ragged B={B} H={H} N={N} d={d} causal={causal}")
    qs, ks, vs = (t.reshape(-1, N, d)[slices] for t in (q, k, v))
    ro, rl = oracle_mod.attention(qs, ks, vs, 1 / math.sqrt(d), causal, rows=rows)
    o, lse = ea.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    sl, rw = torch.tensor(slices, device=o.device), torch.tensor(rows, device=o.device)
    check_bf16(o.reshape(-1, N, d)[sl][:, rw], lse.reshape(-1, N)[sl][:, rw], ro, rl, "fused 8-wave, ragged N")
    assert torch.isfinite(o).all().item()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_unfused_ring_shapes(ea, W, oracle_mod, d, causal):
    # N a multiple of 8 takes the LDS-ring P*V kernel (256 query rows per
    # workgroup, 64-key tiles): one tile, one exact block, ragged rows and keys
    # (264, 520: 8 rows in the last block, 8 keys in the last tile), several
    # blocks.
    for N in [8, 256, 264, 520, 1032]:
        q, k, v = W.make_qkv(1, 2, N, d, torch.bfloat16, seed=300 + N)
        ro, rl = oracle_mod.attention(q, k, v, 1 / math.sqrt(d), causal)
        say(f"[unfused ring] N={N} d={d} causal={causal}")
        o, lse = run(ea, q, k, v, causal, variant="unfused")
        check_bf16(o, lse, ro, rl, "unfused", unfused_lse_tol(q, k, 1 / math.sqrt(d)))


# ---------------------------------------------------------------------------
# Ragged and degenerate shapes, full outputs.
# ---------------------------------------------------------------------------
EDGE_N = [1, 2, 17, 63, 64, 65, 127, 128, 129, 200, 383, 1000]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_shapes_bf16(ea, W, oracle_mod, d, causal):
    for N in EDGE_N:
        q, k, v = W.make_qkv(2, 1, N, d, torch.bfloat16, seed=N)
        ro, rl = oracle_mod.attention(q, k, v, 1 / math.sqrt(d), causal)
        say(f"[edge] bf16 N={N} d={d} causal={causal}")
        o, lse = run(ea, q, k, v, causal)
        check_bf16(o, lse, ro, rl, "fused")
        o, lse = run(ea, q, k, v, causal, variant="unfused")
        check_bf16(o, lse, ro, rl, "unfused", unfused_lse_tol(q, k, 1 / math.sqrt(d)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_shapes_many_slices_bf16(ea, W, oracle_mod, d, causal):
    # With few (batch, head) slices the forward runs the split-key kernel (the
    # shapes above); 130 slices make every N here launch more than 128 blocks
    # of 128 rows, so the regular kernel handles the same ragged lengths.
    slices = [0, 64, 129]
    for N in [17, 129, 200, 1000]:
        q, k, v = W.make_qkv(1, 130, N, d, torch.bfloat16, seed=500 + N)
        qs, ks, vs = (t.reshape(-1, N, d)[slices] for t in (q, k, v))
        ro, rl = oracle_mod.attention(qs, ks, vs, 1 / math.sqrt(d), causal)
        say(f"[edge] bf16 130 slices N={N} d={d} causal={causal}")
        o, lse = run(ea, q, k, v, causal)
        check_bf16(o.reshape(-1, N, d)[slices], lse.reshape(-1, N)[slices], ro, rl, "fused, regular kernel")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_shapes_f32(ea, W, oracle_mod, d, causal):
    for N in [1, 5, 31, 32, 33, 127, 129, 300]:
        q, k, v = W.make_qkv(1, 2, N, d, torch.float32, seed=100 + N)
        ro, rl = oracle_mod.attention(q, k, v, 1 / math.sqrt(d), causal)
        say(f"[edge] fp32 N={N} d={d} causal={causal}")
        o, lse = run(ea, q, k, v, causal)
        check_f32(o, lse, ro, rl, "fused")
        o, lse = run(ea, q, k, v, causal, variant="unfused")
        check_f32(o, lse, ro, rl, "unfused")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_shapes_many_slices_f32(ea, W, oracle_mod, d, causal):
    # Grids of fewer workgroups than compute units (the shapes above) run the
    # split-key fp32 kernel; 260 slices launch at least 260 blocks of 128
    # rows, so the regular kernel sees the same ragged lengths.
    slices = [0, 129, 259]
    for N in [17, 129, 300]:
        q, k, v = W.make_qkv(1, 260, N, d, torch.float32, seed=700 + N)
        qs, ks, vs = (t.reshape(-1, N, d)[slices] for t in (q, k, v))
        ro, rl = oracle_mod.attention(qs, ks, vs, 1 / math.sqrt(d), causal)
        say(f"[edge] fp32 260 slices N={N} d={d} causal={causal}")
        o, lse = run(ea, q, k, v, causal)
        check_f32(o.reshape(-1, N, d)[slices], lse.reshape(-1, N)[slices], ro, rl,
                  "fused, regular kernel")


def test_large_logits_f32(ea, W, oracle_mod):
    # Q x 8 through both fp32 kernels: the split one (2 slices) and the
    # regular one (256 slices, three of them checked).
    for causal in (False, True):
        for H, slices in ((2, [0, 1]), (256, [3, 100, 255])):
            q, k, v = W.make_qkv(1, H, 300, 64, torch.float32, seed=31, q_mult=8.0)
            qs, ks, vs = (t.reshape(-1, 300, 64)[slices] for t in (q, k, v))
            ro, rl = oracle_mod.attention(qs, ks, vs, 1 / 8.0, causal)
            say(f"[edge] fp32 Qx8 H={H} N=300 causal={causal}")
            o, lse = run(ea, q, k, v, causal)
            check_f32(o.reshape(-1, 300, 64)[slices], lse.reshape(-1, 300)[slices], ro, rl,
                      f"fused H={H}")


def test_large_logits_bf16(ea, W, oracle_mod):
    # Q x 8 at a small size: frequent running-max rescales.
    for causal in (False, True):
        q, k, v = W.make_qkv(1, 4, 777, 128, torch.bfloat16, seed=7, q_mult=8.0)
        ro, rl = oracle_mod.attention(q, k, v, 1 / math.sqrt(128), causal)
        say(f"[edge] bf16 Qx8 N=777 causal={causal}")
        o, lse = run(ea, q, k, v, causal)
        check_bf16(o, lse, ro, rl, "fused")


def test_explicit_scale(ea, W, oracle_mod):
    q, k, v = W.make_qkv(1, 2, 300, 64, torch.bfloat16, seed=9)
    for scale in (0.05, 0.3):
        ro, rl = oracle_mod.attention(q, k, v, scale, True)
        o, lse = run(ea, q, k, v, True, scale=scale)
        check_bf16(o, lse, ro, rl, f"fused scale={scale}")


# ---------------------------------------------------------------------------
# Coverage, invariants, determinism, streams.
# ---------------------------------------------------------------------------
def test_every_output_written(ea, W):
    for dtype, fn in ((torch.bfloat16, "attn_fwd"), (torch.float32, "attn_fwd_f32")):
        for causal in (False, True):
            q, k, v = (t.cuda() for t in W.make_qkv(2, 3, 333, 128, dtype, seed=5))
            o = torch.full_like(q, float("nan"))
            lse = torch.full(q.shape[:3], float("nan"), device=q.device)
            getattr(ea, fn)(q, k, v, o, lse, causal=causal)
            torch.cuda.synchronize()
            assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item(), (fn, causal)


def test_ones_values_give_ones(ea, W):
    q, k, _ = W.make_qkv(1, 2, 1000, 128, torch.bfloat16, seed=11)
    v = torch.ones_like(q)
    for causal in (False, True):
        o, _ = run(ea, q, k, v, causal)
        err = (o.float() - 1).abs().max().item()
        say(f"  V=1 causal={causal}: max|O-1|={err:.3e}")
        assert err <= 1e-2


def test_key_permutation_invariance(ea, W):
    q, k, v = W.make_qkv(1, 1, 512, 64, torch.bfloat16, seed=12)
    perm = torch.randperm(512, generator=torch.Generator().manual_seed(0))
    o1, l1 = run(ea, q, k, v, False)
    o2, l2 = run(ea, q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), False)
    assert (o1.float() - o2.float()).abs().max().item() <= BF16_MAX
    assert (l1 - l2).abs().max().item() <= 2 * BF16_LSE  # two results, each within BF16_LSE


def test_deterministic(ea, W):
    q, k, v = (t.cuda() for t in W.make_qkv(2, 4, 1024, 128, torch.bfloat16, seed=13))
    a = ea.attention(q, k, v, causal=True)
    b = ea.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_side_stream_and_no_lse(ea, W, oracle_mod):
    q, k, v = W.make_qkv(1, 2, 256, 64, torch.bfloat16, seed=14)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    s = torch.cuda.Stream()
    o = torch.empty_like(qd)
    with torch.cuda.stream(s):
        ea.attn_fwd(qd, kd, vd, o, None, causal=False, stream=s)
    s.synchronize()
    ro, rl = oracle_mod.attention(q, k, v, 1 / 8, False)
    check_bf16(o.cpu(), rl, ro, rl, "side stream, lse=NULL")


def test_empty_inputs_are_noops(ea):
    q = torch.empty(0, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = ea.attention(q, q, q)
    assert o.numel() == 0
    q = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = ea.attention(q, q, q)
    torch.cuda.synchronize()
    assert o.numel() == 0


def test_rejects_bad_head_dim_on_device(ea):
    q = torch.zeros(1, 1, 16, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ea.AttnError) as ei:
        ea.attention(q, q, q)
    assert ei.value.status == ea.STATUS["ATTN_ERR_HEAD_DIM"]


def test_schedule_independence(ea, W):
    # The same slice computed inside a large batch (eight-wave workgroups,
    # K-ahead pipeline) and in a batch of copies of it small enough for
    # four-wave workgroups visits the same key tiles in the same
    # order for every row, with the same 32-row wave, so the results must agree
    # bit for bit.  Alone, the slice takes the split-key kernel, which sums the
    # keys in another order: it must agree within the bf16 tolerance.
    for B, H, N, causal, copies in ((4, 64, 1024, False, 32), (1, 32, 8192, True, 8)):
        q, k, v = (t.cuda() for t in W.make_qkv(B, H, N, 128, torch.bfloat16, seed=21))
        say(f"[schedule] B={B} H={H} N={N} causal={causal}")
        o_all, l_all = ea.attention(q, k, v, causal=causal)
        for idx in (0, B * H - 1):
            b, h = divmod(idx, H)
            qs, ks, vs = (t[b:b + 1, h:h + 1].contiguous() for t in (q, k, v))
            qc, kc, vc = (t.expand(1, copies, N, 128).contiguous() for t in (qs, ks, vs))
            oc, lc = ea.attention(qc, kc, vc, causal=causal)
            o1, l1 = ea.attention(qs, ks, vs, causal=causal)
            torch.cuda.synchronize()
            for c in (0, copies - 1):
                assert torch.equal(oc[0, c], o_all[b, h]), (B, H, N, causal, idx, c)
                assert torch.equal(lc[0, c], l_all[b, h]), (B, H, N, causal, idx, c)
            d_o = (o1[0, 0].float() - o_all[b, h].float()).abs()
            d_l = (l1[0, 0] - l_all[b, h]).abs().max().item()
            say(f"  split-key vs regular: max|dO|={d_o.max().item():.3e} mean={d_o.mean().item():.3e} "
                f"max|dlse|={d_l:.3e}")
            assert d_o.max().item() <= BF16_MAX and d_o.mean().item() <= BF16_MEAN and d_l <= 2 * BF16_LSE
        del q, k, v, o_all, l_all
        torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1500, 2304, 4100])
def test_persistent_matches_per_block_kernel(ea, W, oracle_mod, causal, N):
    # With the (batch, head) slices a multiple of the XCD count, the 8-wave
    # forward runs persistently (one workgroup per CU walking a list of query
    # blocks, prefetching the next block's Q, K and V); with one slice fewer it
    # launches one workgroup per query block.  Each block is computed the same
    # way in both, so shared slices must agree bit for bit.  N = 4100 gives
    # causal blocks an odd tile count (the next block's first V tile is then
    # loaded after the last barrier), 1500 and 4100 end in a ragged tile.
    B, H, d = 1, 64, 128
    q, k, v = (t.cuda() for t in W.make_qkv(B, H, N, d, torch.bfloat16, seed=1300 + N + causal))
    say(f"[persistent] B={B} H={H} N={N} causal={causal}")
    o_all, l_all = ea.attention(q, k, v, causal=causal)
    o_63, l_63 = ea.attention(q[:, :63].contiguous(), k[:, :63].contiguous(), v[:, :63].contiguous(), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o_all[:, :63], o_63) and torch.equal(l_all[:, :63], l_63)
    rows = sorted({0, 255, 256, N // 2, N - 65, N - 1})
    ro, rl = oracle_mod.attention(q[0, 60:].cpu(), k[0, 60:].cpu(), v[0, 60:].cpu(), 1 / math.sqrt(d), causal,
                                  rows=rows)
    rw = torch.tensor(rows, device=o_all.device)
    check_bf16(o_all[0, 60:][:, rw], l_all[0, 60:][:, rw], ro, rl, "persistent, last slices")


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 20, 4096, 128, False),   # 1.25 rounds of 8-wave workgroups: 4-wave grid
    (1, 24, 2048, 64, False),    # 0.75 rounds: 8-wave (persistent) grid
    (1, 36, 4000, 128, False),   # 2.25 rounds, ragged: 4-wave grid
    (8, 16, 1280, 128, True),    # causal, 1280 keys: 4-wave grid
    (4, 16, 2000, 64, True),     # causal d = 64 up to 2048 keys: 4-wave grid
    (2, 32, 1300, 128, True),    # causal past 1280 keys at d = 128: 8-wave grid
])
def test_launch_shapes_match_oracle(ea, W, oracle_mod, B, H, N, d, causal):
    # The grids the launcher chooses between four- and eight-wave workgroups
    # (both with K one tile ahead), each checked on every row of two slices;
    # the same slice in a grid of copies large enough for eight-wave
    # workgroups must agree bit for bit (same tiles, same order per row).
    q, k, v = (t.cuda() for t in W.make_qkv(B, H, N, d, torch.bfloat16, seed=1500 + N + d))
    say(f"[launch shape] B={B} H={H} N={N} d={d} causal={causal}")
    o, lse = ea.attention(q, k, v, causal=causal)
    torch.cuda.synchronize()
    for idx in (0, B * H - 1):
        b, h = divmod(idx, H)
        ro, rl = oracle_mod.attention(q[b, h].cpu(), k[b, h].cpu(), v[b, h].cpu(), 1 / math.sqrt(d), causal)
        check_bf16(o[b, h], lse[b, h], ro, rl, f"slice {idx}")
    qs, ks, vs = (t[:1, :1].expand(1, 64, N, d).contiguous() for t in (q, k, v))
    o64, l64 = ea.attention(qs, ks, vs, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o64[0, 63], o[0, 0]) and torch.equal(l64[0, 63], lse[0, 0])
