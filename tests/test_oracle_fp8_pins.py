"""Pins for the oracle's 8-bit input path: the E4M3 and E5M2 decoders and
the dequantised attention built on them.

* every one of the 256 codes against torch's own float8_e4m3fn conversion (an
  independent implementation of the OCP format);
* hand-decoded codes from the format definition (bias 7, subnormals, the two
  NaN codes, the largest finite value 448);
* dequantised attention against float64 torch.softmax on torch-dequantised
  inputs, and the placement of the three descale factors;
* planted mistakes in copies of the decoder must each fail a pin;
* the same for E5M2 (torch's float8_e5m2, hand-decoded codes with bias 15,
  the infinities and NaNs of the all-ones exponent, the largest finite value
  57344) and attention over inputs of mixed formats.
"""
import inspect
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_124_amd import workloads as W


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


HAND = {  # code: value, from sign / 4-bit exponent (bias 7) / 3-bit mantissa
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
    0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3C: 1.5, 0x40: 2.0, 0x44: 3.0, 0x78: 256.0, 0x7E: 448.0,
    0xB8: -1.0, 0xC0: -2.0, 0xFE: -448.0, 0x81: -(2.0 ** -9),
}


def _decoder_passes(decode):
    codes = np.arange(256, dtype=np.uint8)
    got = decode(codes)
    if not np.array_equal(got, _torch_decode(codes), equal_nan=True):
        return False
    if any(got[c] != v for c, v in HAND.items()):
        return False
    if not (np.isnan(got[0x7F]) and np.isnan(got[0xFF])):
        return False
    return bool(np.signbit(got[0x80])) and got[0x80] == 0.0


def test_decoder_matches_torch_and_hand_values():
    assert _decoder_passes(oracle.decode_e4m3)


def test_decoder_is_monotone_and_symmetric():
    v = oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    assert np.array_equal(oracle.decode_e4m3(np.arange(0x80, 0xFF, dtype=np.uint8)), -v)


def test_decoder_reads_raw_bytes_of_tensors():
    t = torch.tensor([1.0, -448.0, 2.0 ** -9, 0.0]).to(torch.float8_e4m3fn)
    assert np.array_equal(oracle.decode_e4m3(t), [1.0, -448.0, 2.0 ** -9, 0.0])


def _torch_fp8_attention(q8, k8, v8, qd, kd, vd, scale, causal):
    q, k, v = (t.to(torch.float64) * d for t, d in ((q8, qd), (k8, kd), (v8, vd)))
    s = (q @ k.transpose(-1, -2)) * scale
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    return (torch.softmax(s, -1) @ v).numpy(), torch.logsumexp(s, -1).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 64), (37, 64), (130, 128)])
def test_fp8_attention_matches_float64_torch(causal, N, d):
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(2, 2, N, d, seed=3, q_mult=4.0)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attention_fp8(q8, k8, v8, qd, kd, vd, scale, causal)
    o_t, lse_t = _torch_fp8_attention(q8, k8, v8, qd, kd, vd, scale, causal)
    assert np.abs(o - o_t).max() <= 1e-12 * max(1.0, np.abs(o_t).max())
    assert np.abs(lse - lse_t).max() <= 1e-12 * max(1.0, np.abs(lse_t).max())


def test_descale_placement():
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(1, 2, 50, 64, seed=4)
    s = 0.125
    o, lse = oracle.attention_fp8(q8, k8, v8, qd, kd, vd, s, False)
    # V's factor scales the output and nothing else.
    o2, lse2 = oracle.attention_fp8(q8, k8, v8, qd, kd, 2 * vd, s, False)
    assert np.array_equal(o2, 2 * o) and np.array_equal(lse2, lse)
    # Q's and K's factors enter the scores only through scale * qd * kd.
    o3, lse3 = oracle.attention_fp8(q8, k8, v8, 2 * qd, kd / 2, vd, s, False)
    assert np.abs(o3 - o).max() <= 1e-13 and np.abs(lse3 - lse).max() <= 1e-13
    o4, lse4 = oracle.attention_fp8(q8, k8, v8, 2 * qd, kd, vd, s / 2, False)
    assert np.abs(o4 - o).max() <= 1e-13 and np.abs(lse4 - lse).max() <= 1e-13


def test_generator_uses_the_full_range():
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(1, 1, 256, 64, seed=0)
    for t8, ds, t in zip((q8, k8, v8), (qd, kd, vd), W.make_qkv(1, 1, 256, 64, torch.float32, 0)):
        x = oracle.decode_e4m3(t8)
        assert np.abs(x).max() == 448.0
        # Dequantised values are within half an E4M3 step (2^-4 relative for
        # normals, 2^-10 absolute for subnormals) of the float32 draws.
        ref = t.double().numpy() / ds
        assert np.all(np.abs(x - ref) <= np.maximum(np.abs(ref) * 2.0 ** -4, 2.0 ** -10) * 1.0000001)


MUTANTS = {
    "bias_8": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "no_subnormals": ("np.where(e == 0, sub, normal)", "normal"),
    "subnormal_scale": ("sub = (m / 8.0) * 2.0 ** -6", "sub = (m / 8.0) * 2.0 ** -7"),
    "mantissa_width": ("normal = (1.0 + m / 8.0)", "normal = (1.0 + m / 16.0)"),
    "infinity_codes": ("(e == 0xF) & ((b & 0x7) == 0x7)", "(e == 0xF)"),
    "sign_bit": ("np.where(b & 0x80, -1.0, 1.0)", "np.where(b & 0x40, -1.0, 1.0)"),
}


def _mutant(old, new):
    src = inspect.getsource(oracle.decode_e4m3)
    assert src.count(old) == 1
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    return ns["decode_e4m3"]


def test_unmodified_decoder_source_passes():
    assert _decoder_passes(_mutant("def decode_e4m3", "def decode_e4m3"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_decoder_mistake_is_caught(name):
    assert not _decoder_passes(_mutant(*MUTANTS[name])), name


# ---------------------------------------------------------------------------
# E5M2: the same pins for the second OCP 8-bit format.
# ---------------------------------------------------------------------------
def _torch_decode_e5m2(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e5m2).to(torch.float64).numpy()


HAND_E5M2 = {  # code: value, from sign / 5-bit exponent (bias 15) / 2-bit mantissa
    0x00: 0.0, 0x01: 2.0 ** -16, 0x03: 3 * 2.0 ** -16, 0x04: 2.0 ** -14, 0x07: 1.75 * 2.0 ** -14,
    0x38: 0.5, 0x3C: 1.0, 0x3D: 1.25, 0x3E: 1.5, 0x40: 2.0, 0x42: 3.0, 0x78: 32768.0, 0x7B: 57344.0,
    0xBC: -1.0, 0xC0: -2.0, 0xFB: -57344.0, 0x81: -(2.0 ** -16),
}


def _e5m2_decoder_passes(decode):
    codes = np.arange(256, dtype=np.uint8)
    got = decode(codes)
    if not np.array_equal(got, _torch_decode_e5m2(codes), equal_nan=True):
        return False
    if any(got[c] != v for c, v in HAND_E5M2.items()):
        return False
    if not (got[0x7C] == np.inf and got[0xFC] == -np.inf):
        return False
    if not all(np.isnan(got[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF)):
        return False
    return bool(np.signbit(got[0x80])) and got[0x80] == 0.0


def test_e5m2_decoder_matches_torch_and_hand_values():
    assert _e5m2_decoder_passes(oracle.decode_e5m2)


def test_e5m2_decoder_is_monotone_and_symmetric():
    v = oracle.decode_e5m2(np.arange(0x7C, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    assert np.array_equal(oracle.decode_e5m2(np.arange(0x80, 0xFC, dtype=np.uint8)), -v)


def test_e5m2_decoder_reads_raw_bytes_of_tensors():
    t = torch.tensor([1.0, -57344.0, 2.0 ** -16, 0.0]).to(torch.float8_e5m2)
    assert np.array_equal(oracle.decode_e5m2(t), [1.0, -57344.0, 2.0 ** -16, 0.0])
    assert oracle.fp8_format_of(t) == "e5m2" and oracle.fp8_format_of(t.view(torch.uint8)) == "e4m3"


@pytest.mark.parametrize("formats", [("e5m2",) * 3, ("e4m3", "e4m3", "e5m2"), ("e5m2", "e4m3", "e4m3")])
@pytest.mark.parametrize("causal", [False, True])
def test_mixed_format_attention_matches_float64_torch(formats, causal):
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(2, 2, 37, 64, seed=5, q_mult=4.0, formats=formats)
    assert [oracle.fp8_format_of(t) for t in (q8, k8, v8)] == list(formats)
    scale = 1 / math.sqrt(64)
    o, lse = oracle.attention_fp8(q8, k8, v8, qd, kd, vd, scale, causal)
    o_t, lse_t = _torch_fp8_attention(q8, k8, v8, qd, kd, vd, scale, causal)
    assert np.abs(o - o_t).max() <= 1e-12 * max(1.0, np.abs(o_t).max())
    assert np.abs(lse - lse_t).max() <= 1e-12 * max(1.0, np.abs(lse_t).max())
    # Read as the other format, the same bytes give another function.
    other = tuple("e4m3" if f == "e5m2" else "e5m2" for f in formats)
    o2, _ = oracle.attention_fp8(q8.view(torch.uint8), k8.view(torch.uint8), v8.view(torch.uint8),
                                 qd, kd, vd, scale, causal, formats=other)
    assert not np.allclose(o2, o)


def test_e5m2_generator_uses_the_full_range():
    f = ("e5m2",) * 3
    q8, k8, v8, qd, kd, vd = W.make_qkv_fp8(1, 1, 256, 64, seed=0, formats=f)
    for t8, ds, t in zip((q8, k8, v8), (qd, kd, vd), W.make_qkv(1, 1, 256, 64, torch.float32, 0)):
        x = oracle.decode_e5m2(t8)
        assert np.abs(x).max() == 57344.0
        # Within half an E5M2 step: 2^-3 relative for normals, 2^-17 absolute
        # for subnormals.
        ref = t.double().numpy() / ds
        assert np.all(np.abs(x - ref) <= np.maximum(np.abs(ref) * 2.0 ** -3, 2.0 ** -17) * 1.0000001)


MUTANTS_E5M2 = {
    "bias_16": ("np.exp2(e.astype(np.float64) - 15.0)", "np.exp2(e.astype(np.float64) - 16.0)"),
    "no_subnormals": ("np.where(e == 0, sub, normal)", "normal"),
    "subnormal_scale": ("sub = (m / 4.0) * 2.0 ** -14", "sub = (m / 4.0) * 2.0 ** -15"),
    "mantissa_width": ("normal = (1.0 + m / 4.0)", "normal = (1.0 + m / 8.0)"),
    "exponent_width": ("e = (b >> 2) & 0x1F", "e = (b >> 3) & 0xF"),
    "no_infinity": ("np.where((b & 0x3) == 0, sign * np.inf, np.nan)", "np.nan"),
    "sign_bit": ("np.where(b & 0x80, -1.0, 1.0)", "np.where(b & 0x40, -1.0, 1.0)"),
}


def _mutant_e5m2(old, new):
    src = inspect.getsource(oracle.decode_e5m2)
    assert src.count(old) == 1
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    return ns["decode_e5m2"]


def test_unmodified_e5m2_decoder_source_passes():
    assert _e5m2_decoder_passes(_mutant_e5m2("def decode_e5m2", "def decode_e5m2"))


@pytest.mark.parametrize("name", sorted(MUTANTS_E5M2))
def test_planted_e5m2_decoder_mistake_is_caught(name):
    assert not _e5m2_decoder_passes(_mutant_e5m2(*MUTANTS_E5M2[name])), name
