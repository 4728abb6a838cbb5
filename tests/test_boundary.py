"""C-ABI boundary on the CPU: the library loads, exports what include/attn.h
declares, sizes the unfused workspace as the pages count the score matrix,
and rejects bad arguments with status codes before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
EW_HEADER = os.path.join(ROOT, "include", "ew_chain.h")


@pytest.fixture(scope="module")
def lib():
    import exact_attention_124_amd as ea
    if not os.path.exists(ea.library_path()):
        from exact_attention_124_amd import build
        build.build()
    return ea.load_library()


def declared_functions(header=HEADER, prefix="attn_"):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(" + prefix + r"[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["attn_fwd", "attn_fwd_f32", "attn_fwd_unfused", "attn_fwd_unfused_f32",
                            "attn_unfused_workspace_bytes", "attn_status_string",
                            "attn_last_hip_error", "attn_bwd", "attn_bwd_workspace_bytes", "attn_fwd_fp8", "attn_fwd_masked",
                            "attn_bwd_noalloc", "attn_fwd_fp8_fmt"])


def test_ew_header_declares_the_chain():
    assert declared_functions(EW_HEADER, "ew_") == ["ew_chain_fused", "ew_chain_unfused"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions() + declared_functions(EW_HEADER, "ew_"):
        assert hasattr(lib, name), name
        ctypes.cast(getattr(lib, name), ctypes.c_void_p)


def test_status_strings(lib):
    import exact_attention_124_amd as ea
    for code in range(10):
        s = ea.attn_status_string(code)
        assert s and s != "unknown status"
    assert ea.attn_status_string(99) == "unknown status"
    assert ea.attn_last_hip_error() == 0


@pytest.mark.parametrize("N,expected", [(2048, 8_388_608), (4096, 33_554_432),
                                        (8192, 134_217_728), (16384, 536_870_912)])
def test_workspace_reproduces_per_head_score_sizes(lib, N, expected):
    # "Attention Is Memory-Bound, and Nobody Noticed for Five Years", score-matrix
    # size paragraph: one 16-bit head is 8.4 / 33.6 / 134.2 / 536.9 MB at
    # 2,048 / 4,096 / 8,192 / 16,384 tokens.
    import exact_attention_124_amd as ea
    got = ea.attn_unfused_workspace_bytes(1, 1, N, 2)
    assert got == expected
    assert round(got / 1e6, 1) == {2048: 8.4, 4096: 33.6, 8192: 134.2, 16384: 536.9}[N]


def test_workspace_reproduces_batch_figure_and_traffic(lib):
    # Same page: batch 8 x 32 heads x 8,192 tokens needs 34.4 GB of scores; four
    # crossings are ~138 GB, ~70 ms at ~2 TB/s.
    import exact_attention_124_amd as ea
    s = ea.attn_unfused_workspace_bytes(8, 32, 8192, 2)
    assert s == 34_359_738_368
    assert round(s / 1e9, 1) == 34.4
    assert round(4 * s / 1e9) == 137  # the page rounds 4 x 34.4 up to 138
    assert 65 <= 4 * s / 2e12 * 1e3 <= 70


def test_workspace_edge_cases(lib):
    import exact_attention_124_amd as ea
    assert ea.attn_unfused_workspace_bytes(0, 1, 1, 2) == 0
    assert ea.attn_unfused_workspace_bytes(1, 1, -5, 2) == 0
    assert ea.attn_unfused_workspace_bytes(2**31 - 1, 2**31 - 1, 2**31 - 1, 4) == 0  # overflow
    assert ea.attn_unfused_workspace_bytes(3, 5, 7, 4) == 3 * 5 * 7 * 7 * 4


# Fake, well-separated, aligned device addresses: validation never dereferences them.
A = 1 << 40
GAP = 1 << 36
Q, K, V, O, L, W = (A + i * GAP for i in range(6))


def fwd(lib, name="attn_fwd", q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=256, d=64, scale=0.125,
        causal=0):
    return getattr(lib, name)(q, k, v, o, lse, B, H, N, d, scale, causal, None)


def unf(lib, name="attn_fwd_unfused", ws=W, ws_bytes=None, B=1, H=2, N=256, d=64, elem=2, **kw):
    if ws_bytes is None:
        ws_bytes = B * H * N * N * elem
    args = dict(q=Q, k=K, v=V, o=O, lse=L)
    args.update(kw)
    return getattr(lib, name)(args["q"], args["k"], args["v"], args["o"], args["lse"], ws, ws_bytes,
                              B, H, N, d, 0.125, 0, None)


@pytest.mark.parametrize("name", ["attn_fwd", "attn_fwd_f32"])
def test_validation_codes(lib, name):
    S = {k: v for k, v in __import__("exact_attention_124_amd").STATUS.items()}
    assert fwd(lib, name, q=None) == S["ATTN_ERR_NULL"]
    assert fwd(lib, name, o=None) == S["ATTN_ERR_NULL"]
    assert fwd(lib, name, N=-1) == S["ATTN_ERR_SHAPE"]
    assert fwd(lib, name, B=-2) == S["ATTN_ERR_SHAPE"]
    assert fwd(lib, name, N=0) == S["ATTN_OK"]          # empty: nothing enqueued
    assert fwd(lib, name, H=0, d=3) == S["ATTN_OK"]     # empty wins over other checks
    assert fwd(lib, name, N=0, q=None, k=None, v=None, o=None, lse=None) == S["ATTN_OK"]
    for d in (0, 32, 96, 100, 256):
        assert fwd(lib, name, d=d) == S["ATTN_ERR_HEAD_DIM"]
    assert fwd(lib, name, scale=0.0) == S["ATTN_ERR_ARG"]
    assert fwd(lib, name, scale=-1.0) == S["ATTN_ERR_ARG"]
    assert fwd(lib, name, scale=float("nan")) == S["ATTN_ERR_ARG"]
    assert fwd(lib, name, scale=float("inf")) == S["ATTN_ERR_ARG"]
    assert fwd(lib, name, causal=2) == S["ATTN_ERR_ARG"]
    assert fwd(lib, name, q=Q + 8) == S["ATTN_ERR_ALIGN"]
    assert fwd(lib, name, o=O + 4) == S["ATTN_ERR_ALIGN"]
    assert fwd(lib, name, lse=L + 2) == S["ATTN_ERR_ALIGN"]
    assert fwd(lib, name, o=Q) == S["ATTN_ERR_ALIAS"]
    assert fwd(lib, name, o=V + 4096) == S["ATTN_ERR_ALIAS"]
    assert fwd(lib, name, lse=K + 16) == S["ATTN_ERR_ALIAS"]
    assert fwd(lib, name, lse=O + 256) == S["ATTN_ERR_ALIAS"]
    assert fwd(lib, name, N=1 << 26, d=128) == S["ATTN_ERR_SHAPE"]  # 32-bit slice offsets
    assert fwd(lib, name, B=1 << 16, H=1 << 16) == S["ATTN_ERR_SHAPE"]


@pytest.mark.parametrize("name,elem", [("attn_fwd_unfused", 2), ("attn_fwd_unfused_f32", 4)])
def test_unfused_validation_codes(lib, name, elem):
    S = __import__("exact_attention_124_amd").STATUS
    assert unf(lib, name, elem=elem, ws=None) == S["ATTN_ERR_NULL"]
    assert unf(lib, name, elem=elem, ws_bytes=2 * 256 * 256 * elem - 1) == S["ATTN_ERR_WORKSPACE"]
    assert unf(lib, name, elem=elem, ws=W + 8) == S["ATTN_ERR_ALIGN"]
    assert unf(lib, name, elem=elem, ws=O) == S["ATTN_ERR_ALIAS"]
    assert unf(lib, name, elem=elem, ws=L - 64) == S["ATTN_ERR_ALIAS"]
    assert unf(lib, name, elem=elem, q=None) == S["ATTN_ERR_NULL"]
    assert unf(lib, name, elem=elem, N=0) == S["ATTN_OK"]


def fp8(lib, q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=256, d=64, scale=0.125, qd=0.01, kd=0.02, vd=0.03,
        causal=0):
    return lib.attn_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, qd, kd, vd, causal, None)


def test_fp8_validation_codes(lib):
    S = __import__("exact_attention_124_amd").STATUS
    # Every call below fails validation or is empty: nothing is launched.
    assert fp8(lib, q=None) == S["ATTN_ERR_NULL"]
    assert fp8(lib, N=-1) == S["ATTN_ERR_SHAPE"]
    assert fp8(lib, N=0, q=None, k=None, v=None, o=None, lse=None, qd=float("nan")) == S["ATTN_OK"]
    assert fp8(lib, d=96) == S["ATTN_ERR_HEAD_DIM"]
    for name in ("qd", "kd", "vd", "scale"):
        for bad in (0.0, -1.0, float("nan"), float("inf")):
            assert fp8(lib, **{name: bad}) == S["ATTN_ERR_ARG"], (name, bad)
    assert fp8(lib, causal=2) == S["ATTN_ERR_ARG"]
    assert fp8(lib, k=K + 8) == S["ATTN_ERR_ALIGN"]
    assert fp8(lib, o=O + 2) == S["ATTN_ERR_ALIGN"]
    # q, k, v are 1 byte per element and o 2 bytes: B*H*N*d = 32768 elements.
    assert fp8(lib, o=Q + 32768 - 16) == S["ATTN_ERR_ALIAS"]   # o starts inside q
    assert fp8(lib, o=V - 65536 + 16) == S["ATTN_ERR_ALIAS"]   # o's tail runs into v
    assert fp8(lib, lse=O + 65536 - 4) == S["ATTN_ERR_ALIAS"]  # lse starts inside o
    assert fp8(lib, N=1 << 26, d=128) == S["ATTN_ERR_SHAPE"]   # 32-bit slice offsets of o


def fp8_fmt(lib, fq=0, fk=0, fv=0, q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=256, d=64, scale=0.125, qd=0.01,
            kd=0.02, vd=0.03, causal=0):
    return lib.attn_fwd_fp8_fmt(q, k, v, o, lse, B, H, N, d, scale, qd, kd, vd, fq, fk, fv, causal, None)


def test_fp8_format_validation_codes(lib):
    S = __import__("exact_attention_124_amd").STATUS
    # Every call below fails validation or is empty: nothing is launched.
    for f in (-1, 2, 3, 255):
        assert fp8_fmt(lib, fq=f) == S["ATTN_ERR_ARG"]
        assert fp8_fmt(lib, fk=f) == S["ATTN_ERR_ARG"]
        assert fp8_fmt(lib, fv=f) == S["ATTN_ERR_ARG"]
    assert fp8_fmt(lib, N=0, fq=7) == S["ATTN_OK"]  # empty: a no-op, as every entry point
    assert fp8_fmt(lib, 1, 1, 1, q=None) == S["ATTN_ERR_NULL"]
    assert fp8_fmt(lib, 1, 0, 1, d=96) == S["ATTN_ERR_HEAD_DIM"]
    assert fp8_fmt(lib, 1, 1, 0, qd=0.0) == S["ATTN_ERR_ARG"]
    assert fp8_fmt(lib, 0, 1, 1, o=Q + 16) == S["ATTN_ERR_ALIAS"]
    assert fp8_fmt(lib, 1, 1, 1, k=K + 8) == S["ATTN_ERR_ALIGN"]
    assert "fp8 formats" in lib.attn_status_string(S["ATTN_ERR_ARG"]).decode()


BIAS = A + 10 * GAP


def masked(lib, q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=256, d=64, scale=0.125, causal=0, wl=-1, wr=-1,
           bias=BIAS, sb=0, sh=256 * 256, si=256):
    return lib.attn_fwd_masked(q, k, v, o, lse, B, H, N, d, scale, causal, wl, wr, bias, sb, sh, si, None)


def test_masked_validation_codes(lib):
    S = __import__("exact_attention_124_amd").STATUS
    # Every call below fails validation or is empty: nothing is launched.
    assert masked(lib, q=None) == S["ATTN_ERR_NULL"]
    assert masked(lib, N=0) == S["ATTN_OK"]
    assert masked(lib, d=80) == S["ATTN_ERR_HEAD_DIM"]
    assert masked(lib, causal=5) == S["ATTN_ERR_ARG"]
    assert masked(lib, sb=-4) == S["ATTN_ERR_ARG"]
    assert masked(lib, bias=BIAS + 2) == S["ATTN_ERR_ALIGN"]
    assert masked(lib, si=1 << 25) == S["ATTN_ERR_SHAPE"]          # 32-bit row offsets
    assert masked(lib, bias=O + 1024) == S["ATTN_ERR_ALIAS"]        # bias inside o
    assert masked(lib, bias=L - 16, sh=0, si=0) == S["ATTN_ERR_ALIAS"]  # [N] row runs into lse
    assert masked(lib, o=Q) == S["ATTN_ERR_ALIAS"]


def ew(lib, name, x=Q, y=O, bias=BIAS, rows=64, cols=768, scale=0.5):
    getattr(lib, name).argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_longlong, ctypes.c_int, ctypes.c_float,
                                                            ctypes.c_void_p]
    return getattr(lib, name)(x, y, bias, rows, cols, scale, None)


@pytest.mark.parametrize("name", ["ew_chain_fused", "ew_chain_unfused"])
def test_ew_validation_codes(lib, name):
    S = __import__("exact_attention_124_amd").STATUS
    # Every call below fails validation or is empty: nothing is launched.
    assert ew(lib, name, rows=0) == S["ATTN_OK"]
    assert ew(lib, name, cols=0, x=None) == S["ATTN_OK"]
    assert ew(lib, name, rows=-1) == S["ATTN_ERR_SHAPE"]
    assert ew(lib, name, x=None) == S["ATTN_ERR_NULL"]
    assert ew(lib, name, bias=None) == S["ATTN_ERR_NULL"]
    assert ew(lib, name, cols=770) == S["ATTN_ERR_SHAPE"]
    assert ew(lib, name, scale=float("nan")) == S["ATTN_ERR_ARG"]
    assert ew(lib, name, y=O + 8) == S["ATTN_ERR_ALIGN"]
    assert ew(lib, name, bias=BIAS + 4) == S["ATTN_ERR_ALIGN"]
    assert ew(lib, name, y=Q + 1024) == S["ATTN_ERR_ALIAS"]      # partial overlap
    assert ew(lib, name, bias=O + 64) == S["ATTN_ERR_ALIAS"]     # bias inside y


DO, DQ, DK, DV = (A + i * GAP for i in range(6, 10))


def bwd(lib, ws=W, ws_bytes=None, B=1, H=2, N=256, d=64, **kw):
    if ws_bytes is None:
        ws_bytes = B * H * 2 * ((N + 31) // 32 * 32) * 4
    args = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, scale=0.125, causal=0)
    args.update(kw)
    return lib.attn_bwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["dout"], args["dq"],
                        args["dk"], args["dv"], ws, ws_bytes, B, H, N, d, args["scale"], args["causal"], None)


def test_bwd_workspace_bytes(lib):
    import exact_attention_124_amd as ea
    assert ea.attn_bwd_workspace_bytes(1, 1, 1) == 2 * 32 * 4
    assert ea.attn_bwd_workspace_bytes(2, 3, 33) == 2 * 3 * 2 * 64 * 4
    assert ea.attn_bwd_workspace_bytes(8, 32, 8192) == 8 * 32 * 2 * 8192 * 4
    assert ea.attn_bwd_workspace_bytes(0, 1, 1) == 0
    assert ea.attn_bwd_workspace_bytes(1, 1, -1) == 0


def test_bwd_validation_codes(lib):
    S = __import__("exact_attention_124_amd").STATUS
    # Every call below fails validation, so nothing is launched on the fake
    # addresses (a fully valid call would enqueue kernels).
    for name in ("q", "o", "lse", "dout", "dq", "dk", "dv"):
        assert bwd(lib, **{name: None}) == S["ATTN_ERR_NULL"], name
    assert bwd(lib, ws=None) == S["ATTN_ERR_NULL"]
    assert bwd(lib, N=0) == S["ATTN_OK"]
    assert bwd(lib, N=-1) == S["ATTN_ERR_SHAPE"]
    assert bwd(lib, d=96) == S["ATTN_ERR_HEAD_DIM"]
    assert bwd(lib, scale=0.0) == S["ATTN_ERR_ARG"]
    assert bwd(lib, causal=3) == S["ATTN_ERR_ARG"]
    assert bwd(lib, dq=DQ + 8) == S["ATTN_ERR_ALIGN"]
    assert bwd(lib, ws=W + 4) == S["ATTN_ERR_ALIGN"]
    assert bwd(lib, ws_bytes=2 * 2 * 256 * 4 - 1) == S["ATTN_ERR_WORKSPACE"]
    assert bwd(lib, dq=Q) == S["ATTN_ERR_ALIAS"]        # output over an input
    assert bwd(lib, dk=DO + 64) == S["ATTN_ERR_ALIAS"]
    assert bwd(lib, dv=DQ) == S["ATTN_ERR_ALIAS"]       # two outputs
    assert bwd(lib, ws=L) == S["ATTN_ERR_ALIAS"]        # workspace over lse
    assert bwd(lib, ws=DK + 32) == S["ATTN_ERR_ALIAS"]  # workspace over an output
    assert bwd(lib, N=1 << 26, d=128) == S["ATTN_ERR_SHAPE"]


def bwd_noalloc(lib, B=1, H=2, N=256, d=64, **kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, scale=0.125, causal=0)
    args.update(kw)
    return lib.attn_bwd_noalloc(args["q"], args["k"], args["v"], args["o"], args["lse"], args["dout"],
                                args["dq"], args["dk"], args["dv"], B, H, N, d, args["scale"], args["causal"],
                                None)


def test_bwd_noalloc_validation_codes(lib):
    # The checks of attn_bwd without the workspace ones, then the static
    # scratch limit (16 MiB of statistics: B*H*round_up(N, 32) <= 2^21 rows).
    # Every call below fails validation or is empty: nothing is launched.
    import exact_attention_124_amd as ea
    S = ea.STATUS
    for name in ("q", "o", "lse", "dout", "dq", "dk", "dv"):
        assert bwd_noalloc(lib, **{name: None}) == S["ATTN_ERR_NULL"], name
    assert bwd_noalloc(lib, N=0) == S["ATTN_OK"]
    assert bwd_noalloc(lib, N=-1) == S["ATTN_ERR_SHAPE"]
    assert bwd_noalloc(lib, d=96) == S["ATTN_ERR_HEAD_DIM"]
    assert bwd_noalloc(lib, scale=0.0) == S["ATTN_ERR_ARG"]
    assert bwd_noalloc(lib, dq=DQ + 8) == S["ATTN_ERR_ALIGN"]
    assert bwd_noalloc(lib, dq=Q) == S["ATTN_ERR_ALIAS"]
    assert bwd_noalloc(lib, dv=DQ) == S["ATTN_ERR_ALIAS"]
    # one padded row past the limit: 2^21 + 32 rows of statistics
    assert ea.attn_bwd_workspace_bytes(1, 64, 32768) == ea.BWD_SCRATCH_BYTES
    assert bwd_noalloc(lib, B=1, H=64, N=32768 + 1) == S["ATTN_ERR_SCRATCH"]
    assert bwd_noalloc(lib, B=8, H=32, N=16384, d=128) == S["ATTN_ERR_SCRATCH"]
    assert "scratch" in ea.attn_status_string(S["ATTN_ERR_SCRATCH"])


def test_python_binding_rejects_cpu_tensors(lib):
    import torch
    import exact_attention_124_amd as ea
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.attention(x, x, x)


def test_python_binding_names_what_is_wrong(lib):
    # Every rejection happens before any GPU call, so CPU tensors exercise it.
    import torch
    import exact_attention_124_amd as ea
    x = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    o = torch.empty_like(x)
    with pytest.raises(TypeError, match="k must be a torch.Tensor"):
        ea.attn_fwd(x, x.numpy, x, o)
    with pytest.raises(TypeError, match="v must be torch.bfloat16"):
        ea.attn_fwd(x, x, x.float(), o)
    with pytest.raises(TypeError, match="q must be torch.float32"):
        ea.attn_fwd_f32(x, x, x, o)
    with pytest.raises(ValueError, match="k must be a contiguous"):
        ea.attn_fwd(x, x.transpose(2, 3), x, o)
    with pytest.raises(ValueError, match="q must be a contiguous"):
        ea.attn_fwd(x[0], x[0], x[0], o)
    with pytest.raises(ValueError, match="must live on a GPU"):
        ea.attn_fwd(x, x, x, o)
    with pytest.raises(TypeError, match="q must be torch.float8_e4m3fn"):
        ea.attn_fwd_fp8(x, x, x, o, None, 1.0, 1.0, 1.0)
    with pytest.raises(ValueError, match="lse .* is required"):
        ea.attn_bwd_noalloc(x, x, x, o, None, x, o, o, o)


def test_no_oracle_in_product_path():
    # The product package neither imports nor links the oracle.
    pkg = os.path.join(ROOT, "exact_attention_124_amd")
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle)|liboracle|attn_oracle", re.M)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not pat.search(text), f"{f} refers to the oracle"
