"""attn_bwd_noalloc against attn_bwd through the C ABI.

Both run the same three kernels; only where the per-row statistics live
differs (the library's static per-GPU scratch array instead of a caller
workspace).  The results must be bitwise identical.  Two calls in a row, the
second with a smaller problem, check that the scratch's leftover contents from
the first call do not leak into the second; a call at exactly the scratch
limit (B*H*round_up(N, 32) = 2^21 rows) and one past it are checked too.
"""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu


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


def _inputs(W, B, H, N, d, causal, seed):
    q, k, v = (t.cuda() for t in W.make_qkv(B, H, N, d, torch.bfloat16, seed=seed))
    dout = W.make_grad(B, H, N, d, torch.bfloat16, seed=seed).cuda()
    return q, k, v, dout


def _compare(ea, q, k, v, dout, causal):
    o, lse = ea.attention(q, k, v, causal=causal)
    ref = ea.attention_backward(q, k, v, o, lse, dout, causal=causal)
    got = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    ea.attn_bwd_noalloc(q, k, v, o, lse, dout, *got, causal=causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(a).all().item(), name
        assert torch.equal(a, b), name


def test_noalloc_matches_workspace_entry_point(ea):
    from exact_attention_124_amd import workloads as W
    for (B, H, N, d, causal, seed) in ((2, 4, 1000, 128, True, 61), (1, 2, 300, 64, False, 62)):
        say(f"[noalloc] B={B} H={H} N={N} d={d} causal={causal}")
        q, k, v, dout = _inputs(W, B, H, N, d, causal, seed)
        _compare(ea, q, k, v, dout, causal)


def test_noalloc_at_the_scratch_limit(ea):
    from exact_attention_124_amd import workloads as W
    B, H, N, d = 8, 32, 8192, 128  # 2^21 rows of statistics: exactly the 16 MiB scratch
    assert ea.attn_bwd_workspace_bytes(B, H, N) == ea.BWD_SCRATCH_BYTES
    say(f"[noalloc] at the limit B={B} H={H} N={N} d={d}")
    q, k, v, dout = _inputs(W, B, H, N, d, False, 63)
    _compare(ea, q, k, v, dout, False)
    del q, k, v, dout
    torch.cuda.empty_cache()
    # one padded row block more is rejected before anything is enqueued
    big = torch.empty(1, 64, 32768 + 1, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, 64, 32768 + 1, dtype=torch.float32, device="cuda")
    outs = [torch.empty_like(big) for _ in range(5)]
    with pytest.raises(ea.AttnError) as ei:
        ea.attn_bwd_noalloc(big, outs[0], outs[1], outs[2], lse, outs[3], outs[4], torch.empty_like(big),
                            torch.empty_like(big))
    assert ei.value.status == ea.STATUS["ATTN_ERR_SCRATCH"]
