"""fp64 CPU oracle for scaled dot-product attention.

Test infrastructure, not product code: only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it.  The HIP library neither imports nor links anything here, and this package
imports nothing from the HIP library.

The attention arithmetic lives in plain C, fp64: ``attn_oracle.c`` (the
textbook forward: scores, row max, exp-sum, weighted values),
``attn_bwd_oracle.c`` (its gradients), ``attn_probs_oracle.c`` (rows of the
probability matrix) and ``attn_masked_oracle.c`` (forward with window masks
and an additive bias).  This module builds them with gcc and marshals numpy
arrays through ctypes; the e4m3 and e5m2 decoding and the elementwise chain
(relu(scale * x + bias)) are written out here in numpy.

Definition followed: grasp.study lesson on standard self-attention, section
"The Computational Steps of Standard Self-Attention" (scores = Q K^T, row-wise
softmax, output = P V), with the exactness claim of "Attention Is
Memory-Bound, and Nobody Noticed for Five Years" (the fused method returns the
same function up to floating-point reassociation).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "attn_oracle.c"), os.path.join(_HERE, "attn_bwd_oracle.c"),
         os.path.join(_HERE, "attn_probs_oracle.c"), os.path.join(_HERE, "attn_masked_oracle.c")]
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def _stale() -> bool:
    return not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(s) for s in _SRCS)


def build(force: bool = True) -> str:
    """Compile the oracle C sources into ``liboracle.so`` with gcc (fp64, no
    FMA contraction, OpenMP over rows).  Returns the library path."""
    if not force and not _stale():
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra", *_SRCS, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _stale():
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    lib.oracle_attn_f64.restype = ctypes.c_int
    lib.oracle_attn_f64.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,   # q k v
        ctypes.c_void_p, ctypes.c_void_p,                    # o lse
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,      # S N d
        ctypes.c_double, ctypes.c_int,                       # scale causal
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,       # rows n_rows threads
    ]
    lib.oracle_attn_bwd_f64.restype = ctypes.c_int
    lib.oracle_attn_bwd_f64.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # q k v dout
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,                   # dq dk dv
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,                      # S N d
        ctypes.c_double, ctypes.c_int,                                       # scale causal
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,    # qrows n_q krows n_k
        ctypes.c_int,                                                        # threads
    ]
    lib.oracle_attn_probs_f64.restype = ctypes.c_int
    lib.oracle_attn_probs_f64.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,   # q k w
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,      # S N d
        ctypes.c_double, ctypes.c_int,                       # scale causal
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,       # rows n_rows threads
    ]
    lib.oracle_attn_masked_f64.restype = ctypes.c_int
    lib.oracle_attn_masked_f64.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,   # q k v bias
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,                      # sb sh si
        ctypes.c_void_p, ctypes.c_void_p,                                    # o lse
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,      # B H N d
        ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,       # scale causal wl wr
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,                       # rows n_rows threads
    ]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def max_threads() -> int:
    """OpenMP threads the oracle uses by default."""
    return int(_load().oracle_max_threads())


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: exact upcast on the CPU
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def attention(q, k, v, scale: float, causal: bool = False, rows=None, threads: int = 0):
    """Exact attention in fp64.

    ``q``, ``k``, ``v``: arrays of shape ``[..., N, d]`` (any leading dims are
    flattened into independent slices).  ``rows``: optional 1-D sequence of
    query-row indices to compute (every slice); ``None`` = all rows.
    Returns ``(o, lse)`` with shapes ``[..., R, d]`` and ``[..., R]``.
    """
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    if not (q64.shape == k64.shape == v64.shape) or q64.ndim < 2:
        raise ValueError("q, k, v must share one shape [..., N, d]")
    lead = q64.shape[:-2]
    N, d = q64.shape[-2:]
    S = int(np.prod(lead)) if lead else 1
    if rows is None:
        R = N
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
        R = rows_arr.size
    o = np.empty((S, R, d), dtype=np.float64)
    lse = np.empty((S, R), dtype=np.float64)
    rc = _load().oracle_attn_f64(
        q64.ctypes.data, k64.ctypes.data, v64.ctypes.data,
        o.ctypes.data, lse.ctypes.data,
        S, N, d, float(scale), 1 if causal else 0,
        rows_arr.ctypes.data if rows_arr is not None else None,
        R if rows_arr is not None else 0, int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_f64 failed with code {rc}")
    return o.reshape(*lead, R, d), lse.reshape(*lead, R)


def probabilities(q, k, scale: float, causal: bool = False, rows=None, threads: int = 0):
    """The attention weights softmax(scale * q k^T) of the selected query rows
    (every row if ``rows`` is None), fp64, shape ``[..., R, N]``; disallowed
    (causal) keys get 0."""
    q64, k64 = _as_f64(q), _as_f64(k)
    if q64.shape != k64.shape or q64.ndim < 2:
        raise ValueError("q and k must share one shape [..., N, d]")
    lead = q64.shape[:-2]
    N, d = q64.shape[-2:]
    S = int(np.prod(lead)) if lead else 1
    r = _index(rows)
    R = N if r is None else r.size
    w = np.empty((S, R, N), dtype=np.float64)
    rc = _load().oracle_attn_probs_f64(q64.ctypes.data, k64.ctypes.data, w.ctypes.data, S, N, d, float(scale),
                                       1 if causal else 0, r.ctypes.data if r is not None else None,
                                       R if r is not None else 0, int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_probs_f64 failed with code {rc}")
    return w.reshape(*lead, R, N)


# ---------------------------------------------------------------------------
# 8-bit floating point inputs.
# ---------------------------------------------------------------------------
def decode_e4m3(codes) -> np.ndarray:
    """Value of each OCP FP8 E4M3 byte as float64, written out from the format
    definition: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 encodes subnormals m * 2^-9; the all-ones exponent with
    all-ones mantissa (0x7F, 0xFF) is NaN and every other code is finite (no
    infinities), so the largest value is 1.75 * 2^8 = 448.

    ``codes``: uint8 array, or a torch float8_e4m3fn / uint8 tensor (read as
    raw bytes, never converted by torch)."""
    if hasattr(codes, "detach"):
        import torch
        t = codes.detach().to("cpu").contiguous()
        if t.dtype != torch.uint8:
            t = t.view(torch.uint8)
        codes = t.numpy()
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((b & 0x7) == 0x7), np.nan, val)


def decode_e5m2(codes) -> np.ndarray:
    """Value of each OCP FP8 E5M2 byte as float64, written out from the format
    definition: 1 sign bit, 5 exponent bits with bias 15, 2 mantissa bits;
    exponent field 0 encodes subnormals m * 2^-16; the all-ones exponent
    encodes infinity with a zero mantissa (0x7C, 0xFC) and NaN otherwise, so
    the largest finite value is 1.75 * 2^15 = 57344.

    ``codes``: uint8 array, or a torch float8_e5m2 / uint8 tensor (read as raw
    bytes, never converted by torch)."""
    if hasattr(codes, "detach"):
        import torch
        t = codes.detach().to("cpu").contiguous()
        if t.dtype != torch.uint8:
            t = t.view(torch.uint8)
        codes = t.numpy()
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 2) & 0x1F
    m = (b & 0x3).astype(np.float64)
    normal = (1.0 + m / 4.0) * np.exp2(e.astype(np.float64) - 15.0)
    sub = (m / 4.0) * 2.0 ** -14
    val = sign * np.where(e == 0, sub, normal)
    special = np.where((b & 0x3) == 0, sign * np.inf, np.nan)
    return np.where(e == 0x1F, special, val)


FP8_FORMATS = ("e4m3", "e5m2")


def fp8_format_of(t) -> str:
    """``"e5m2"`` for a torch float8_e5m2 tensor, else ``"e4m3"``."""
    return "e5m2" if str(getattr(t, "dtype", "")) == "torch.float8_e5m2" else "e4m3"


def decode_fp8(codes, fmt: str) -> np.ndarray:
    """:func:`decode_e4m3` or :func:`decode_e5m2` by ``fmt``."""
    if fmt not in FP8_FORMATS:
        raise ValueError(f"unknown fp8 format {fmt!r}")
    return decode_e4m3(codes) if fmt == "e4m3" else decode_e5m2(codes)


def dequantize_fp8(t8, descale: float, fmt: str | None = None) -> np.ndarray:
    """``descale * decode(t8)`` in fp64 (exact); the format is ``fmt``, else
    that of ``t8``'s torch dtype."""
    return decode_fp8(t8, fmt or fp8_format_of(t8)) * float(np.float32(descale))


def attention_fp8(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float, scale: float,
                  causal: bool = False, rows=None, threads: int = 0, formats=None):
    """Exact attention of dequantised 8-bit inputs: the inputs are
    ``descale * decode(code)`` per tensor (exact in fp64: a 4- or 3-bit
    significand times an fp32 factor), then :func:`attention` in fp64.
    ``formats``: (q, k, v) formats, each ``"e4m3"`` or ``"e5m2"``; by default
    each tensor's torch dtype decides (anything but float8_e5m2 is E4M3)."""
    fq, fk, fv = formats if formats is not None else (fp8_format_of(q8), fp8_format_of(k8), fp8_format_of(v8))
    return attention(dequantize_fp8(q8, q_descale, fq), dequantize_fp8(k8, k_descale, fk),
                     dequantize_fp8(v8, v_descale, fv), scale, causal, rows=rows, threads=threads)


def attention_masked(q, k, v, scale: float, causal: bool = False, window_left: int = -1,
                     window_right: int = -1, bias=None, rows=None, threads: int = 0):
    """Exact attention with a causal / sliding-window mask and an additive
    bias, fp64.  ``q``, ``k``, ``v``: ``[B, H, N, d]``.  ``bias``: None, or an
    array broadcastable to ``[B, H, N, N]`` (added to the scaled scores; -inf
    removes a key).  A window side < 0 is unbounded.  Rows with no allowed
    finite score give o = 0 and lse = -inf.  Returns ``(o, lse)`` shaped
    ``[B, H, R, d]`` and ``[B, H, R]``."""
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    if not (q64.shape == k64.shape == v64.shape) or q64.ndim != 4:
        raise ValueError("q, k, v must share one shape [B, H, N, d]")
    B, H, N, d = q64.shape
    if bias is not None:
        b64 = _as_f64(bias)
        if b64.ndim != 4 or b64.shape[2:] != (N, N) or b64.shape[0] not in (1, B) or b64.shape[1] not in (1, H):
            raise ValueError("bias must be [B|1, H|1, N, N]")
        b64 = np.ascontiguousarray(b64)
        sb = 0 if b64.shape[0] == 1 else b64.shape[1] * N * N
        sh = 0 if b64.shape[1] == 1 else N * N
        si = N
    else:
        b64, sb, sh, si = None, 0, 0, 0
    r = _index(rows)
    R = N if r is None else r.size
    o = np.empty((B, H, R, d), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    rc = _load().oracle_attn_masked_f64(
        q64.ctypes.data, k64.ctypes.data, v64.ctypes.data, b64.ctypes.data if b64 is not None else None,
        sb, sh, si, o.ctypes.data, lse.ctypes.data, B, H, N, d, float(scale), 1 if causal else 0,
        int(window_left), int(window_right), r.ctypes.data if r is not None else None,
        R if r is not None else 0, int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_masked_f64 failed with code {rc}")
    return o, lse


# ---------------------------------------------------------------------------
# Elementwise chain (the fusion example of the pages).
# ---------------------------------------------------------------------------
def elementwise_chain(x, scale: float, bias):
    """y = relu(scale * x + bias) in fp64, element by element, for a
    ``[rows, cols]`` array ``x`` and a ``[cols]`` bias broadcast over rows:
    multiply by a scalar, add a bias, apply an activation ("Attention Is
    Memory-Bound, and Nobody Noticed for Five Years", the elementwise-chain
    paragraph; ReLU is the reading of "an activation").  Also returns the two
    intermediate tensors ``(t1, t2)`` = (scale * x, t1 + bias)."""
    x64 = _as_f64(x)
    b64 = _as_f64(bias)
    if x64.ndim != 2 or b64.shape != (x64.shape[1],):
        raise ValueError("x must be [rows, cols] and bias [cols]")
    t1 = float(np.float32(scale)) * x64
    t2 = t1 + b64[None, :]
    y = np.where(t2 > 0.0, t2, 0.0)
    return y, t1, t2


def _index(idx):
    if idx is None:
        return None
    return np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1))


def attention_backward(q, k, v, dout, scale: float, causal: bool = False, rows=None, keys=None,
                       threads: int = 0):
    """Exact gradient of attention in fp64 for an upstream gradient ``dout``.

    ``q``, ``k``, ``v``, ``dout``: arrays of shape ``[..., N, d]``.  ``rows``:
    optional query-row indices for ``dq``; ``keys``: optional key indices for
    ``dk`` and ``dv`` (the same indices in every slice).  Returns
    ``(dq, dk, dv)`` shaped ``[..., Rq, d]``, ``[..., Rk, d]``, ``[..., Rk, d]``.
    """
    q64, k64, v64, g64 = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    if not (q64.shape == k64.shape == v64.shape == g64.shape) or q64.ndim < 2:
        raise ValueError("q, k, v, dout must share one shape [..., N, d]")
    lead = q64.shape[:-2]
    N, d = q64.shape[-2:]
    S = int(np.prod(lead)) if lead else 1
    qr, kr = _index(rows), _index(keys)
    Rq = N if qr is None else qr.size
    Rk = N if kr is None else kr.size
    dq = np.empty((S, Rq, d), dtype=np.float64)
    dk = np.empty((S, Rk, d), dtype=np.float64)
    dv = np.empty((S, Rk, d), dtype=np.float64)
    rc = _load().oracle_attn_bwd_f64(
        q64.ctypes.data, k64.ctypes.data, v64.ctypes.data, g64.ctypes.data,
        dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, S, N, d, float(scale), 1 if causal else 0,
        qr.ctypes.data if qr is not None else None, Rq if qr is not None else 0,
        kr.ctypes.data if kr is not None else None, Rk if kr is not None else 0, int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_bwd_f64 failed with code {rc}")
    return dq.reshape(*lead, Rq, d), dk.reshape(*lead, Rk, d), dv.reshape(*lead, Rk, d)
