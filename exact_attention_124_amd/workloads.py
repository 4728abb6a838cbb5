"""Seeded synthetic workloads for attention forward.

This module draws inputs and picks which slices/rows to check.  It holds none
of attention's arithmetic, so the HIP path and the fp64 oracle can both be fed
from it without sharing any computation.

Recipe (the pages name no data; these shapes follow the score-matrix sizes and
head dimensions the pages discuss, "d is 64 or 128", and a 12-head model):

* ``torch.Generator('cpu').manual_seed(seed)``, then ``Q``, ``K``, ``V`` drawn
  in that order as float32 ``randn`` of shape ``[B, H, N, d]``;
* ``Q`` multiplied by ``q_mult`` (8 for the long-context stress case, a power
  of two, so exact before or after rounding);
* converted to the working dtype with ``Tensor.to`` (round to nearest even for
  bfloat16);
* slices to check against the oracle: ``randperm(B*H)`` from a second
  generator seeded with ``seed + 1``;
* the upstream gradient dO of the backward: float32 ``randn`` of the same
  shape from a generator seeded with ``seed + 100``, then the working dtype;
* additive attention bias: float32 ``randn`` of shape ``[Bb, Hb, N, N]`` from
  a generator seeded with ``seed + 200``, times ``scale``, with a fraction
  ``drop`` of entries (never a diagonal one) set to -inf, chosen by a second
  generator seeded with ``seed + 201``;
* elementwise chain: x float32 ``randn`` ``[rows, cols]`` rounded to bf16
  and a float32 ``randn`` bias ``[cols]``, from a generator seeded with
  ``seed + 300`` (x first);
* 8-bit inputs: the float32 ``Q``, ``K``, ``V`` above, each divided by its
  per-tensor factor ``descale = max|x| / 448`` (float32) and converted to
  ``torch.float8_e4m3fn`` (round to nearest even; the largest magnitude lands
  on 448, the largest finite E4M3 value); for a tensor requested in E5M2,
  ``descale = max|x| / 57344`` and ``torch.float8_e5m2``.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: torch.dtype
    causal: bool
    q_mult: float = 1.0
    oracle_slices: int | None = None   # None = every (b, h) slice
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Dense-contraction FLOP convention: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def elem_bytes(self) -> int:
        return torch.tensor([], dtype=self.dtype).element_size()

    def describe(self) -> str:
        dt = {torch.bfloat16: "bf16", torch.float32: "fp32"}[self.dtype]
        mask = "causal" if self.causal else "non-causal"
        extra = f", Q x{self.q_mult:g}" if self.q_mult != 1.0 else ""
        return f"{mask} attention fwd B={self.B} H={self.H} N={self.N} d={self.d} {dt}{extra}"


# The five workloads, smallest first.
WORKLOADS = {
    "small_fp32": Workload("small_fp32", 1, 1, 128, 64, torch.float32, False),
    "gpt2_heads_bf16": Workload("gpt2_heads_bf16", 1, 12, 1024, 64, torch.bfloat16, False),
    "causal_2k_bf16": Workload("causal_2k_bf16", 4, 32, 2048, 128, torch.bfloat16, True),
    "dense_8k_bf16": Workload("dense_8k_bf16", 8, 32, 8192, 128, torch.bfloat16, False,
                              oracle_slices=4),
    "causal_32k_qx8_bf16": Workload("causal_32k_qx8_bf16", 1, 32, 32768, 128, torch.bfloat16,
                                    True, q_mult=8.0, oracle_slices=2),
}
ORDER = ["small_fp32", "gpt2_heads_bf16", "causal_2k_bf16", "dense_8k_bf16",
         "causal_32k_qx8_bf16"]


def make_qkv(B: int, H: int, N: int, d: int, dtype=torch.bfloat16, seed: int = 0,
             q_mult: float = 1.0, device="cpu"):
    """Draw Q, K, V as described in the module docstring."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if q_mult != 1.0:
        q.mul_(q_mult)
    out = []
    for t in (q, k, v):
        t = t.to(dtype)
        out.append(t.to(device) if str(device) != "cpu" else t)
    return tuple(out)


def make_bias(Bb: int, Hb: int, N: int, seed: int = 0, scale: float = 1.0, drop: float = 0.0, device="cpu"):
    """Additive bias [Bb, Hb, N, N] (see the module docstring)."""
    g = torch.Generator(device="cpu").manual_seed(seed + 200)
    b = torch.randn((Bb, Hb, N, N), generator=g, dtype=torch.float32) * scale
    if drop > 0:
        g2 = torch.Generator(device="cpu").manual_seed(seed + 201)
        m = torch.rand((Bb, Hb, N, N), generator=g2) < drop
        m &= ~torch.eye(N, dtype=torch.bool)
        b.masked_fill_(m, float("-inf"))
    return b.to(device) if str(device) != "cpu" else b


def make_chain(rows: int, cols: int, seed: int = 0, device="cpu"):
    """x (bf16 [rows, cols]) and bias (float32 [cols]) of the elementwise chain."""
    g = torch.Generator(device="cpu").manual_seed(seed + 300)
    x = torch.randn((rows, cols), generator=g, dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn((cols,), generator=g, dtype=torch.float32)
    if str(device) != "cpu":
        x, b = x.to(device), b.to(device)
    return x, b


E4M3_MAX = 448.0


E5M2_MAX = 57344.0
FP8_DTYPES = {"e4m3": (torch.float8_e4m3fn, E4M3_MAX), "e5m2": (torch.float8_e5m2, E5M2_MAX)}


def make_qkv_fp8(B: int, H: int, N: int, d: int, seed: int = 0, q_mult: float = 1.0, device="cpu",
                 formats=("e4m3", "e4m3", "e4m3")):
    """8-bit Q, K, V and their float32 dequantisation factors (see the module
    docstring), in the (q, k, v) ``formats`` ("e4m3" or "e5m2"): returns
    ``(q8, k8, v8, q_descale, k_descale, v_descale)``."""
    qkv = make_qkv(B, H, N, d, torch.float32, seed, q_mult)
    out, scales = [], []
    for t, fmt in zip(qkv, formats):
        dtype, fmax = FP8_DTYPES[fmt]
        amax = float(t.abs().max()) if t.numel() else 1.0
        ds = torch.tensor(amax / fmax if amax > 0 else 1.0, dtype=torch.float32)
        t8 = (t / ds).to(dtype)
        out.append(t8.to(device) if str(device) != "cpu" else t8)
        scales.append(float(ds))
    return (*out, *scales)


def make_grad(B: int, H: int, N: int, d: int, dtype=torch.bfloat16, seed: int = 0, device="cpu"):
    """Upstream gradient dO for the backward (see the module docstring)."""
    g = torch.Generator(device="cpu").manual_seed(seed + 100)
    t = torch.randn((B, H, N, d), generator=g, dtype=torch.float32).to(dtype)
    return t.to(device) if str(device) != "cpu" else t


def workload_inputs(w: Workload, device="cpu"):
    return make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.q_mult, device)


def check_slices(w: Workload) -> list[int]:
    """Flattened (b*H + h) slice indices the oracle checks for workload ``w``."""
    n = w.B * w.H
    if w.oracle_slices is None or w.oracle_slices >= n:
        return list(range(n))
    g = torch.Generator(device="cpu").manual_seed(w.seed + 1)
    return torch.randperm(n, generator=g)[: w.oracle_slices].tolist()


def sample_rows(N: int, count: int, seed: int = 2) -> list[int]:
    """``count`` distinct seeded query rows in [0, N), always including the
    first and the last row (the causal extremes), sorted."""
    if count >= N:
        return list(range(N))
    g = torch.Generator(device="cpu").manual_seed(seed)
    picks = set(torch.randperm(N, generator=g)[: max(count - 2, 0)].tolist())
    picks.update({0, N - 1})
    return sorted(picks)
