"""Exact fused attention forward for MI355X (gfx950).

Thin Python binding over the C ABI in ``include/attn.h`` (``libattn.so``):
argument marshalling only.  Every step of the computation runs in the HIP
kernels of that library; PyTorch supplies device memory and the stream.  If
the library has not been built, every call raises -- there is no fallback.

Functions with the C names take caller-allocated tensors, exactly like the C
entry points; ``attention`` and ``attention_unfused`` allocate the outputs.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "AttnError", "library_path", "load_library", "attn_fwd", "attn_fwd_f32", "attn_fwd_unfused",
    "attn_fwd_unfused_f32", "attn_unfused_workspace_bytes", "attn_status_string",
    "attn_last_hip_error", "attention", "attention_unfused", "STATUS", "attn_bwd",
    "attn_bwd_workspace_bytes", "attention_backward", "attn_fwd_fp8", "attention_fp8",
    "attn_fwd_masked", "attention_masked", "ew_chain_fused", "ew_chain_unfused", "elementwise_chain",
    "attn_bwd_noalloc", "BWD_SCRATCH_BYTES", "attn_fwd_fp8_fmt", "FP8_FORMATS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libattn.so")
_lib = None

# attn_status values (include/attn.h)
STATUS = {
    "ATTN_OK": 0, "ATTN_ERR_NULL": 1, "ATTN_ERR_SHAPE": 2, "ATTN_ERR_HEAD_DIM": 3,
    "ATTN_ERR_ALIGN": 4, "ATTN_ERR_ALIAS": 5, "ATTN_ERR_WORKSPACE": 6, "ATTN_ERR_HIP": 7,
    "ATTN_ERR_ARG": 8, "ATTN_ERR_SCRATCH": 9,
}
# ATTN_BWD_SCRATCH_BYTES (include/attn.h): attn_bwd_noalloc's static statistics buffer per GPU
BWD_SCRATCH_BYTES = 16 << 20
# ATTN_FP8_E4M3 / ATTN_FP8_E5M2 (include/attn.h): input formats of attn_fwd_fp8_fmt
FP8_FORMATS = {"e4m3": 0, "e5m2": 1}


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {attn_status_string(status)} (status {status})"
        if status == STATUS["ATTN_ERR_HIP"]:
            msg += f", hipError_t {attn_last_hip_error()}"
        super().__init__(msg)


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load ``libattn.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m exact_attention_124_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    fwd = [P, P, P, P, P, I, I, I, I, F, I, P]
    unf = [P, P, P, P, P, P, SZ, I, I, I, I, F, I, P]
    for name, args in (("attn_fwd", fwd), ("attn_fwd_f32", fwd),
                       ("attn_fwd_unfused", unf), ("attn_fwd_unfused_f32", unf)):
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = I
    LL = ctypes.c_longlong
    lib.attn_fwd_masked.argtypes = [P, P, P, P, P, I, I, I, I, F, I, I, I, P, LL, LL, LL, P]
    lib.attn_fwd_masked.restype = I
    for name in ("ew_chain_fused", "ew_chain_unfused"):
        fn = getattr(lib, name)
        fn.argtypes = [P, P, P, LL, I, F, P]
        fn.restype = I
    lib.attn_fwd_fp8.argtypes = [P, P, P, P, P, I, I, I, I, F, F, F, F, I, P]
    lib.attn_fwd_fp8.restype = I
    lib.attn_fwd_fp8_fmt.argtypes = [P, P, P, P, P, I, I, I, I, F, F, F, F, I, I, I, I, P]
    lib.attn_fwd_fp8_fmt.restype = I
    lib.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, SZ, I, I, I, I, F, I, P]
    lib.attn_bwd.restype = I
    lib.attn_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P]
    lib.attn_bwd_noalloc.restype = I
    lib.attn_bwd_workspace_bytes.argtypes = [I, I, I]
    lib.attn_bwd_workspace_bytes.restype = SZ
    lib.attn_unfused_workspace_bytes.argtypes = [I, I, I, I]
    lib.attn_unfused_workspace_bytes.restype = SZ
    lib.attn_status_string.argtypes = [I]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = I
    _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_last_hip_error() -> int:
    return int(load_library().attn_last_hip_error())


def attn_unfused_workspace_bytes(B: int, H: int, N: int, elem_bytes: int) -> int:
    return int(load_library().attn_unfused_workspace_bytes(B, H, N, elem_bytes))


def attn_bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, H, N))


# ---------------------------------------------------------------------------
# Marshalling helpers (torch is only a container for device memory here).
# They run on every call, so the accepted case costs a few attribute reads;
# a failed check drops to a slow path that names what is wrong.
# ---------------------------------------------------------------------------
_T = None            # the torch module, imported on first use
_get_device = None   # index of the current device
_raw_stream = None   # raw handle of a device's current stream


def _torch():
    global _T, _get_device, _raw_stream
    if _T is None:
        import torch
        _get_device = torch._C._cuda_getDevice
        _raw_stream = torch._C._cuda_getCurrentRawStream
        _T = torch
    return _T


def _qkv_error(names, tensors, dtype):
    torch = _torch()
    pairs = list(zip(names, tensors))
    for name, t in pairs:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
    for name, t in pairs:
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    for name, t in pairs:
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    for name, t in pairs:
        if not t.is_cuda:
            raise ValueError(f"{name} must live on a GPU")
    if any(t.shape != tensors[0].shape for t in tensors):
        raise ValueError(f"{', '.join(names)} must have the same shape")
    raise ValueError(f"{', '.join(names)} must be on the same device")


def _check_qkv(q, k, v, dtype, names=("q", "k", "v")):
    """(B, H, N, d, device index) of three contiguous, same-shape
    [B, H, N, d] GPU tensors of ``dtype`` on one device; raises otherwise."""
    try:
        shape = q.shape
        if (q.dtype is dtype and k.dtype is dtype and v.dtype is dtype and q.is_cuda
                and len(shape) == 4 and k.shape == shape and v.shape == shape
                and q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
            dev = q.get_device()
            if k.get_device() == dev and v.get_device() == dev:
                B, H, N, d = shape
                return B, H, N, d, dev
    except AttributeError:
        pass
    _qkv_error(names, (q, k, v), dtype)


def _check_out(o, lse, B, H, N, d, dtype, dev, name="o"):
    """``o``: contiguous [B, H, N, d] of ``dtype`` on device ``dev``;
    ``lse`` (if given): contiguous float32 [B, H, N] on the same device."""
    try:
        ok = (o.dtype is dtype and o.shape == (B, H, N, d) and o.is_contiguous()
              and o.get_device() == dev)
    except AttributeError:
        ok = False
    if not ok:
        raise ValueError(f"{name} must be a contiguous {dtype} [B, H, N, d] tensor like q, on q's device")
    if lse is not None:
        try:
            ok = (lse.dtype is _torch().float32 and lse.shape == (B, H, N) and lse.is_contiguous()
                  and lse.get_device() == dev)
        except AttributeError:
            ok = False
        if not ok:
            raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")


def _stream(stream, dev):
    """Raw stream handle: the device's current stream when ``stream`` is
    None, else an int handle or a torch stream's handle."""
    if stream is None:
        if _raw_stream is None:
            _torch()
        return _raw_stream(dev)
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _launch(dev, fn, *args):
    """Call a C entry point with device ``dev`` current: its kernels are
    launched on the current device, which must own the tensors and the
    stream.  The device is switched (and restored) only when another one is
    current."""
    if _get_device is None:
        _torch()
    if dev == _get_device():
        return fn(*args)
    with _T.cuda.device(dev):
        return fn(*args)


def _fwd(name, dtype, q, k, v, o, lse, causal, scale, stream):
    B, H, N, d, dev = _check_qkv(q, k, v, dtype)
    _check_out(o, lse, B, H, N, d, dtype, dev)
    st = _launch(dev, getattr(_lib or load_library(), name), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                 o.data_ptr(), None if lse is None else lse.data_ptr(), B, H, N, d,
                 _scale(scale, d), 1 if causal else 0, _stream(stream, dev))
    if st != 0:
        raise AttnError(st, name)


def _workspace_bytes(workspace, dev):
    """Size in bytes of a contiguous workspace tensor on device ``dev``."""
    try:
        ok = workspace.get_device() == dev and workspace.is_contiguous()
    except AttributeError:
        ok = False
    if not ok:
        raise ValueError("workspace must be a contiguous tensor on q's device")
    return workspace.numel() * workspace.element_size()


def _unfused(name, dtype, elem, q, k, v, o, lse, workspace, causal, scale, stream):
    B, H, N, d, dev = _check_qkv(q, k, v, dtype)
    _check_out(o, lse, B, H, N, d, dtype, dev)
    nbytes = _workspace_bytes(workspace, dev)
    fn = getattr(load_library(), name)
    st = _launch(dev, fn, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse),
                 workspace.data_ptr(), nbytes, B, H, N, d, _scale(scale, d), 1 if causal else 0,
                 _stream(stream, dev))
    if st != 0:
        raise AttnError(st, name)


# ---------------------------------------------------------------------------
# Same names as the C entry points.
# ---------------------------------------------------------------------------
def attn_fwd(q, k, v, o, lse=None, causal=False, scale=None, stream=None):
    """bf16 fused forward into caller-allocated ``o`` (and ``lse``)."""
    _fwd("attn_fwd", _torch().bfloat16, q, k, v, o, lse, causal, scale, stream)


def attn_fwd_f32(q, k, v, o, lse=None, causal=False, scale=None, stream=None):
    """fp32 fused forward into caller-allocated ``o`` (and ``lse``)."""
    _fwd("attn_fwd_f32", _torch().float32, q, k, v, o, lse, causal, scale, stream)


def attn_fwd_unfused(q, k, v, o, lse, workspace, causal=False, scale=None, stream=None):
    """bf16 unfused forward (scores and probabilities in ``workspace``)."""
    _unfused("attn_fwd_unfused", _torch().bfloat16, 2, q, k, v, o, lse, workspace, causal, scale,
             stream)


def attn_fwd_unfused_f32(q, k, v, o, lse, workspace, causal=False, scale=None, stream=None):
    """fp32 unfused forward (scores and probabilities in ``workspace``)."""
    _unfused("attn_fwd_unfused_f32", _torch().float32, 4, q, k, v, o, lse, workspace, causal,
             scale, stream)


def _fp8_formats(q, k, v):
    """ATTN_FP8_* code of each of q, k, v from its torch dtype
    (float8_e4m3fn: E4M3, float8_e5m2: E5M2); raises for any other."""
    torch = _torch()
    codes = {torch.float8_e4m3fn: FP8_FORMATS["e4m3"], torch.float8_e5m2: FP8_FORMATS["e5m2"]}
    out = []
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype not in codes:
            raise TypeError(f"{name} must be torch.float8_e4m3fn or torch.float8_e5m2, got {t.dtype}")
        out.append(codes[t.dtype])
    return out


def _fwd_fp8(name, q, k, v, o, lse, q_descale, k_descale, v_descale, formats, causal, scale, stream):
    torch = _torch()
    u8 = torch.uint8
    B, H, N, d, dev = _check_qkv(q.view(u8), k.view(u8), v.view(u8), u8)
    _check_out(o, lse, B, H, N, d, torch.bfloat16, dev)
    lib = load_library()
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse), B, H, N, d, _scale(scale, d),
            float(q_descale), float(k_descale), float(v_descale)]
    if name == "attn_fwd_fp8_fmt":
        args += [int(f) for f in formats]
    st = _launch(dev, getattr(lib, name), *args, 1 if causal else 0, _stream(stream, dev))
    if st != 0:
        raise AttnError(st, name)


def attn_fwd_fp8(q, k, v, o, lse, q_descale, k_descale, v_descale, causal=False, scale=None, stream=None):
    """fp8 fused forward into caller-allocated bf16 ``o`` (and ``lse``).  Each
    of q, k, v is a torch float8_e4m3fn (OCP E4M3) or float8_e5m2 (OCP E5M2)
    tensor; all E4M3 calls the C ``attn_fwd_fp8``, any E5M2 input
    ``attn_fwd_fp8_fmt`` with the three formats."""
    formats = _fp8_formats(q, k, v)
    name = "attn_fwd_fp8" if not any(formats) else "attn_fwd_fp8_fmt"
    _fwd_fp8(name, q, k, v, o, lse, q_descale, k_descale, v_descale, formats, causal, scale, stream)


def attn_fwd_fp8_fmt(q, k, v, o, lse, q_descale, k_descale, v_descale, q_format, k_format, v_format,
                     causal=False, scale=None, stream=None):
    """The C ``attn_fwd_fp8_fmt``: q, k, v are 1-byte tensors (uint8 or
    either float8 dtype) whose bytes are read in the given formats
    (``FP8_FORMATS["e4m3"]`` or ``FP8_FORMATS["e5m2"]``)."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.element_size() != 1:
            raise TypeError(f"{name} must be a tensor of 1-byte elements")
    _fwd_fp8("attn_fwd_fp8_fmt", q, k, v, o, lse, q_descale, k_descale, v_descale,
             (q_format, k_format, v_format), causal, scale, stream)


def _bias_view(bias, B, H, N, dev):
    """(pointer, stride_b, stride_h, stride_i) of a float32 bias broadcastable
    to [B, H, N, N]: shape [N, N] or [B|1, H|1, N, N], last stride 1."""
    torch = _torch()
    if bias is None:
        return None, 0, 0, 0
    if not isinstance(bias, torch.Tensor) or bias.dtype != torch.float32 or bias.get_device() != dev:
        raise TypeError("bias must be a float32 tensor on q's device")
    if bias.dim() == 2:
        bias = bias.unsqueeze(0).unsqueeze(0)
    if bias.dim() != 4 or tuple(bias.shape[2:]) != (N, N) or bias.shape[0] not in (1, B) \
            or bias.shape[1] not in (1, H) or bias.stride(3) != 1:
        raise ValueError("bias must be [N, N] or [B|1, H|1, N, N] with unit stride along keys")
    sb = 0 if bias.shape[0] == 1 else bias.stride(0)
    sh = 0 if bias.shape[1] == 1 else bias.stride(1)
    return bias.data_ptr(), sb, sh, bias.stride(2)


def attn_fwd_masked(q, k, v, o, lse=None, causal=False, window=(-1, -1), bias=None, scale=None, stream=None):
    """bf16 fused forward with a causal / sliding-window mask and an optional
    float32 additive bias, into caller-allocated ``o`` (and ``lse``).
    ``window`` = (left, right); a negative side is unbounded."""
    torch = _torch()
    B, H, N, d, dev = _check_qkv(q, k, v, torch.bfloat16)
    _check_out(o, lse, B, H, N, d, torch.bfloat16, dev)
    bp, sb, sh, si = _bias_view(bias, B, H, N, dev)
    wl, wr = (int(window[0]), int(window[1]))
    st = _launch(dev, load_library().attn_fwd_masked,
                 q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse),
                 B, H, N, d, _scale(scale, d), 1 if causal else 0, wl, wr, bp, sb, sh, si,
                 _stream(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_fwd_masked")


def _ew(name, x, y, bias, scale, stream):
    torch = _torch()
    for nm, t in (("x", x), ("y", y)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_contiguous() \
                or t.device.type != "cuda":
            raise ValueError(f"{nm} must be a contiguous bf16 [rows, cols] tensor on a GPU")
    dev = x.get_device()
    if y.shape != x.shape or y.get_device() != dev:
        raise ValueError("y must have x's shape and device")
    if not isinstance(bias, torch.Tensor) or bias.dtype != torch.float32 or tuple(bias.shape) != (x.shape[1],) \
            or not bias.is_contiguous() or bias.get_device() != dev:
        raise ValueError("bias must be a contiguous float32 [cols] tensor on x's device")
    st = _launch(dev, getattr(load_library(), name),
                 x.data_ptr(), y.data_ptr(), bias.data_ptr(), x.shape[0], x.shape[1],
                 float(scale), _stream(stream, dev))
    if st != 0:
        raise AttnError(st, name)


def ew_chain_fused(x, y, bias, scale, stream=None):
    """y = relu(scale * x + bias) in one launch (bf16 x, y; float32 bias)."""
    _ew("ew_chain_fused", x, y, bias, scale, stream)


def ew_chain_unfused(x, y, bias, scale, stream=None):
    """The same chain as three launches, each reading and writing the tensor."""
    _ew("ew_chain_unfused", x, y, bias, scale, stream)


def elementwise_chain(x, bias, scale, fused=True, stream=None):
    """Allocating form of ew_chain_fused / ew_chain_unfused."""
    y = _torch().empty_like(x)
    (ew_chain_fused if fused else ew_chain_unfused)(x, y, bias, scale, stream)
    return y


def _check_bwd(q, k, v, o, lse, dout, dq, dk, dv):
    """(B, H, N, d, device index) for the backward's tensors: bf16 q, k, v,
    o, dout, dq, dk, dv of one [B, H, N, d] shape and float32 lse [B, H, N],
    all contiguous on one GPU."""
    if lse is None:
        raise ValueError("lse (the forward's log-sum-exp) is required")
    bf16 = _torch().bfloat16
    B, H, N, d, dev = _check_qkv(q, k, v, bf16)
    _check_out(o, lse, B, H, N, d, bf16, dev)
    for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_out(t, None, B, H, N, d, bf16, dev, name)
    return B, H, N, d, dev


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal=False, scale=None, stream=None):
    """bf16 backward into caller-allocated ``dq``, ``dk``, ``dv``."""
    B, H, N, d, dev = _check_bwd(q, k, v, o, lse, dout, dq, dk, dv)
    nbytes = _workspace_bytes(workspace, dev)
    st = _launch(dev, load_library().attn_bwd,
                 q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                 dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                 workspace.data_ptr(), nbytes,
                 B, H, N, d, _scale(scale, d), 1 if causal else 0, _stream(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_bwd")


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal=False, scale=None, stream=None):
    """bf16 backward into caller-allocated ``dq``, ``dk``, ``dv`` with the
    statistics in the library's static per-GPU scratch (no workspace, no
    allocation).  Calls that overlap on one GPU race on that scratch."""
    B, H, N, d, dev = _check_bwd(q, k, v, o, lse, dout, dq, dk, dv)
    st = _launch(dev, load_library().attn_bwd_noalloc,
                 q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                 dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                 B, H, N, d, _scale(scale, d), 1 if causal else 0, _stream(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_bwd_noalloc")


# ---------------------------------------------------------------------------
# Allocating conveniences.
# ---------------------------------------------------------------------------
def attention(q, k, v, causal=False, scale=None, stream=None):
    """Fused forward; returns ``(o, lse)``.  bf16 or fp32 by ``q.dtype``."""
    torch = _torch()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if q.dtype == torch.bfloat16:
        attn_fwd(q, k, v, o, lse, causal, scale, stream)
    elif q.dtype == torch.float32:
        attn_fwd_f32(q, k, v, o, lse, causal, scale, stream)
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return o, lse


def attention_fp8(q, k, v, q_descale, k_descale, v_descale, causal=False, scale=None, stream=None):
    """fp8 fused forward (each input E4M3 or E5M2 by its torch dtype); returns
    ``(o, lse)`` with ``o`` in bf16."""
    torch = _torch()
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_fwd_fp8(q, k, v, o, lse, q_descale, k_descale, v_descale, causal, scale, stream)
    return o, lse


def attention_masked(q, k, v, causal=False, window=(-1, -1), bias=None, scale=None, stream=None):
    """Masked / biased fused forward; returns ``(o, lse)``."""
    torch = _torch()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_fwd_masked(q, k, v, o, lse, causal, window, bias, scale, stream)
    return o, lse


def attention_unfused(q, k, v, causal=False, scale=None, stream=None, workspace=None):
    """Unfused forward; returns ``(o, lse, workspace)`` (workspace holds P)."""
    torch = _torch()
    B, H, N, _ = q.shape
    elem = 2 if q.dtype == torch.bfloat16 else 4
    if workspace is None:
        workspace = torch.empty(attn_unfused_workspace_bytes(B, H, N, elem), dtype=torch.uint8,
                                device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if q.dtype == torch.bfloat16:
        attn_fwd_unfused(q, k, v, o, lse, workspace, causal, scale, stream)
    elif q.dtype == torch.float32:
        attn_fwd_unfused_f32(q, k, v, o, lse, workspace, causal, scale, stream)
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return o, lse, workspace


def attention_backward(q, k, v, o, lse, dout, causal=False, scale=None, stream=None, workspace=None):
    """Backward of ``attention``; returns ``(dq, dk, dv)`` (bf16)."""
    torch = _torch()
    B, H, N, _ = q.shape
    if workspace is None:
        workspace = torch.empty(max(attn_bwd_workspace_bytes(B, H, N), 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, scale, stream)
    return dq, dk, dv
