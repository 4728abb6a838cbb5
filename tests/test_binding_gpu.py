"""The Python binding on device tensors: each argument check that needs GPU
tensors to reach, and the three ways of naming the stream (current stream,
a torch stream, a raw handle), which must give the same bytes."""
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


def _qkv(B=1, H=2, N=200, d=64, dtype=torch.bfloat16, seed=0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return [torch.randn(B, H, N, d, generator=g).to(dtype).cuda() for _ in range(3)]


def test_rejects_mismatched_device_tensors(ea):
    say("binding checks on GPU tensors")
    q, k, v = _qkv()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="same shape"):
        ea.attn_fwd(q, k[:, :, :100].contiguous(), v, o, lse)
    with pytest.raises(ValueError, match="o must be"):
        ea.attn_fwd(q, k, v, o[:, :, :100].contiguous(), lse)
    with pytest.raises(ValueError, match="o must be"):
        ea.attn_fwd(q, k, v, o.cpu(), lse)
    with pytest.raises(ValueError, match="o must be"):
        ea.attn_fwd(q, k, v, o.float(), lse)
    with pytest.raises(ValueError, match="lse must be"):
        ea.attn_fwd(q, k, v, o, lse.double())
    with pytest.raises(ValueError, match="lse must be"):
        ea.attn_fwd(q, k, v, o, lse[:, :, :100].contiguous())
    with pytest.raises(ValueError, match="lse must be"):
        ea.attn_fwd(q, k, v, o, lse.cpu())
    ws = torch.empty(ea.attn_unfused_workspace_bytes(1, 2, 200, 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="workspace"):
        ea.attn_fwd_unfused(q, k, v, o, lse, ws)
    with pytest.raises(TypeError, match="bias"):
        ea.attn_fwd_masked(q, k, v, o, lse, bias=torch.zeros(200, 200))
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    with pytest.raises(ValueError, match="dout must be"):
        ea.attn_bwd_noalloc(q, k, v, o, lse, q[:, :1].contiguous(), dq, dk, dv)
    with pytest.raises(ValueError, match="dk must be"):
        ea.attn_bwd_noalloc(q, k, v, o, lse, q, dq, dk.float(), dv)
    torch.cuda.synchronize()


def test_stream_forms_agree(ea):
    say("binding stream forms, B=1 H=2 N=200 d=64")
    q, k, v = _qkv(seed=3)
    outs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for form in ("current", "torch", "raw", "side"):
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        if form == "current":
            ea.attn_fwd(q, k, v, o, lse, causal=True)
        elif form == "torch":
            ea.attn_fwd(q, k, v, o, lse, causal=True, stream=torch.cuda.current_stream())
        elif form == "raw":
            ea.attn_fwd(q, k, v, o, lse, causal=True, stream=torch.cuda.current_stream().cuda_stream)
        else:
            with torch.cuda.stream(side):
                ea.attn_fwd(q, k, v, o, lse, causal=True)  # the side stream is current here
            torch.cuda.current_stream().wait_stream(side)
        outs.append((o, lse))
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])
